#!/usr/bin/env python3
"""Benchmark: SparseX prefill on the 32K RAG mix, one MI355X.

Workload: a 32-layer Llama-3-8B-shaped attention stack in bf16 (hidden 4096,
32 q / 8 kv heads, head_dim 128, RoPE theta 5e5) over one request made of a
reused 512-token system segment, 16 reused 1920-token passages and a
256-token new query (31,488 tokens).  Layers 0-3 run full attention; the
Sparse-Q estimation at layer 3 selects 10% of the reused tokens; layers 4-31
realign, recompute the active rows and run sparse attention.  Inputs are
seeded synthetic values (no dataset, random weights), resident in HBM before
timing starts.

A step is one prefill pass of the batch through all 32 layers.  The headline
value is prefill tokens/s per sparse layer: T / t_layer with t_layer = the
wall time from just before the selection to the end of the last sparse layer
(HIP events on the launch stream) / 28.  --pipelined runs the sparse layers
on two streams.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --sweep      (chat32k: time per pass vs threshold)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s per layer @32K (sparse recompute); attn % of MFMA bf16 peak"
METRIC_QWEN = "prefill tokens/s per layer @128K (sparse recompute); attn % of MFMA bf16 peak"
METRIC_1L = "prefill tokens/s, one Llama-3-8B-shaped layer at 4.3K (sparse recompute); attn % of MFMA bf16 peak"
METRIC_AGENT = "prefill tokens/s, one layer, 4 x ~64K agent batch (sparse recompute); attn % of MFMA bf16 peak"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_rag32k_traffic.json")
ATTN_SRC = os.path.join(ROOT, "segment_level_kv_amd", "csrc", "attention.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=["rag32k", "qwen128k", "agent64k", "llama1l"], default="rag32k",
                    help="rag32k (the metric's workload, default); qwen128k: Qwen2.5-7B shapes, "
                         "32 reused 4,000-token segments + 1,024 new tokens, 28 layers, threshold 8; "
                         "agent64k: Llama shapes, 4 requests of ~64K tokens from a pool of 64 "
                         "segments, ratios 5-30%, one layer (selection inside it); llama1l: 8 x 512 "
                         "reused + 256 new tokens, ratio 15%, one layer")
    ap.add_argument("--layers", type=int, default=None, help="default 32 (rag32k) / 28 (qwen128k)")
    ap.add_argument("--threshold", type=int, default=None, help="default 4 (rag32k) / 8 (qwen128k)")
    ap.add_argument("--pipelined", action="store_true",
                    help="run the sparse layers on two streams (layer l+1's realign and recompute "
                         "while layer l attends)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the rag32k line: the chat32k workload at thresholds "
                         "0/10/15/20%% of the layers, plus full recompute and ratio 0%%")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain elementwise copy (torch.neg) of this many MiB of fp32 "
                         "before the timed region, as the byte-counter reference for rocprofv3")
    return ap.parse_args()


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per sparse-attention launch from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("attention_hip_sha256_16") != source_hash(ATTN_SRC):
        return None
    return t.get("bytes_per_launch")


def decode_measure(run, dims, n_layers: int, t: int, reps: int = 5):
    """Decode attention of the request's last token over each sparse layer's
    mixed cache after the prefill (sx_decode_attn), outside the timed prefill
    steps.  Every layer has its own 64 MB K + 64 MB V pool, so a pass over the
    sparse layers streams 3.6 GB and no layer's cache is still on chip when it
    is read again.  Bytes per call: K and V of all tokens and kv heads, plus
    q and o."""
    import torch
    T = run.n_tok
    hq, hkv, d = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    n_req = run.n_req
    q = torch.randn((n_req, hq, d), generator=g, device="cuda").to(torch.bfloat16)
    o = torch.empty((n_req, hq * d), dtype=torch.bfloat16, device="cuda")
    layers = list(range(t, n_layers))
    for l in layers:
        run.decode_attention(l, q, o)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        for l in layers:
            run.decode_attention(l, q, o)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (reps * len(layers))
    nbytes = 2.0 * T * hkv * d * 2 + 2.0 * 2 * n_req * hq * d
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "sx_decode_attn (decode_fwd + decode_merge)", "tokens": T,
            "us_per_call": round(us, 2), "bytes_per_call": nbytes, "achieved_GBps": round(gbs, 1),
            "peak_GBps": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
            "calls_timed": reps * len(layers)}


def mfma_peak_measure(shapes=((256, 3000), (2048, 400), (8192, 100)), reps: int = 5):
    """Measured bf16 MFMA throughput (sx_mfma_peak_probe: back-to-back
    v_mfma_f32_32x32x16_bf16 on every compute unit), timed with events on the
    launch stream, outside the timed prefill steps, with constant operands
    and with random bf16 operands.  The best of a few launch shapes is the
    measured peak of each kind (the highest rate the chip was seen to
    sustain).  256 workgroups is the attention's occupancy (two waves per
    SIMD).  Random operands make the chip draw more power and hold a lower
    clock: that rate is what an MFMA-bound kernel on the benchmark's random
    data can reach at best."""
    import torch
    from segment_level_kv_amd import _lib as L
    res = {}
    for kind, rnd in (("constant_operands", False), ("random_operands", True)):
        rates = []
        for n_wg, iters in shapes:
            out = torch.empty(n_wg * 8, dtype=torch.float32, device="cuda")
            L.sx_mfma_peak_probe(n_wg, iters, out, random_operands=rnd)
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                L.sx_mfma_peak_probe(n_wg, iters, out, random_operands=rnd)
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / reps
            flops = float(n_wg) * 8 * iters * 16 * 32768
            rates.append({"workgroups": n_wg, "iters": iters, "ms_per_launch": round(ms, 4),
                          "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)})
        res[kind] = {"TFLOP/s": max(r["TFLOP/s"] for r in rates), "shapes": rates}
    return {"kernel": "sx_mfma_peak_probe (v_mfma_f32_32x32x16_bf16, 8 waves per workgroup)",
            "TFLOP/s": res["constant_operands"]["TFLOP/s"],
            "random_operands_TFLOP/s": res["random_operands"]["TFLOP/s"],
            "constant_operands": res["constant_operands"], "random_operands": res["random_operands"],
            "spec_TFLOP/s": PEAK_BF16_TFLOPS}


def cpu_baseline(dims, plan, n_sparse: int, T: int, reused: int, seed: int = 4242):
    """The float64 oracle on a bounded sample of one sparse layer of the same
    workload, scaled to tokens/s per layer.  Sample (about 10 s of CPU work
    per repetition on 16 cores): realign of 16 of the 1920-token passages,
    projection of 1024 active rows, attention of 2048 active rows, and 128
    Sparse-Q rows of the selection probe (amortised over the sparse layers);
    each part is timed best of 3 and scaled by its share of the layer's
    work."""
    n_pass, n_rec, n_att, n_probe = 16, 1024, 2048, 128
    import oracle
    from segment_level_kv_amd import synth
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        cores = max([p.get("num_threads", 1) for p in info] or [1])
        if info:
            blas = " / ".join(f"{p.get('internal_api', '?')} {p.get('version', '')}".strip() for p in info)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1

    def best_of(fn, reps=3):
        best = float("inf")
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            best = min(best, time.perf_counter() - t0)
        return best
    rng = np.random.default_rng(seed)
    hkv, hq, d = dims.n_kv_heads, dims.n_q_heads, dims.head_dim
    sq = plan["sq_rows"].astype(np.int64)
    cand = np.flatnonzero(plan["tok_class"] == 0)
    k = int(plan["k"][0])
    S = np.sort(rng.choice(cand, size=k, replace=False))
    A = np.union1d(sq, S)
    R = reused
    K = synth.to_storage(rng.standard_normal((T, hkv, d)), "bf16")
    V = synth.to_storage(rng.standard_normal((T, hkv, d)), "bf16")
    t = {}
    # realign: n_pass passages, each moved by its own offset
    def realign():
        for i in range(n_pass):
            a = 512 + 1920 * i
            oracle.realign_segment(K[a:a + 1920], V[a:a + 1920], a, 2048 + 1920 * i, dims.theta, "bf16")
    t["realign"] = best_of(realign) * (R / (1920 * n_pass))
    # recompute: n_rec rows
    x = synth.to_storage(synth._rmsnormed_gaussian(rng, n_rec, dims.hidden, dims.eps), "bf16")
    wq, wk, wv = synth._weights(rng, dims)
    t["recompute"] = best_of(lambda: oracle.project_rows(x, wq, wk, wv, S[:n_rec], dims.theta, hq, hkv,
                                                         d, "bf16")) * (len(A) / n_rec)
    # attention: n_att active rows, scaled by key count
    rows = np.sort(rng.choice(A, size=n_att, replace=False))
    q = synth.to_storage(rng.standard_normal((n_att, hq, d)), "bf16")
    t["attn"] = best_of(lambda: oracle.causal_attention(q, rows, K, V)) * (np.sum(A + 1) / np.sum(rows + 1))
    # selection probe: n_probe Sparse-Q rows (LSE + scores), amortised
    qs = synth.to_storage(rng.standard_normal((n_probe, hq, d)), "bf16")
    def probe():
        _, lse = oracle.causal_attention(qs, sq[:n_probe], K, V)
        oracle.attention_mass_scores(qs, sq[:n_probe], K, lse)
    t["select"] = best_of(probe) * (len(sq) / n_probe) / n_sparse
    sample_s = sum(t_ * f for t_, f in zip(
        (t["realign"], t["recompute"], t["attn"], t["select"]),
        (1920 * n_pass / R, n_rec / len(A), np.sum(rows + 1) / np.sum(A + 1),
         n_probe * n_sparse / len(sq))))
    layer_s = sum(t.values())
    return {"value": T / layer_s, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "blas_vendor": blas, "repeats": "best of 3 per part",
            "sample": (f"float64 NumPy oracle, one sparse layer of the same workload: realign of "
                       f"{n_pass} 1920-token passages (x R/{1920 * n_pass}), projection of {n_rec} "
                       f"active rows (x |A|/{n_rec}), attention of {n_att} active rows (x key-count "
                       f"share), {n_probe} Sparse-Q probe rows (x {len(sq)}/{n_probe}, amortised "
                       f"over the sparse layers); each part timed best of 3"),
            "sample_cpu_seconds": round(float(sample_s), 2),
            "seconds_per_layer": layer_s, "parts_s": {k_: round(float(v), 4) for k_, v in t.items()}}


def sweep(args):
    """The chat workload (instruction | reused history | the history's last,
    uncached partial block | question) through the full+sparse hybrid stack
    at several thresholds t (the trade-off of §3.4 and Table 1): one prefill
    pass of 32 layers, timed with HIP events, per configuration."""
    import torch
    from segment_level_kv_amd import synth
    from segment_level_kv_amd.stack import HybridStackRun
    dims = synth.LLAMA8B
    seg_lengths, layout, p_src = synth.chat_layout()
    seg_len = {i: n for i, n in enumerate(seg_lengths)}
    seg_p = {i: p for i, p in enumerate(p_src)}
    n_layers = args.layers if args.layers is not None else 32
    T = sum(seg_len[v] if k == "reuse" else v for k, v in layout)
    n_cache = sum(seg_lengths)
    ratio = (10, 100)
    configs = [("full recompute", n_layers, ratio)]
    for frac in (0.0, 0.10, 0.15, 0.20):
        configs.append((f"t={int(frac * 100)}%", int(round(frac * n_layers)), ratio))
    configs.append(("ratio 0%, t=0", 0, (0, 100)))
    points = []
    for name, t, rt in configs:
        inputs = synth.TorchStackInputs(2005, dims, n_layers, T, n_cache, t, "cuda")
        run = HybridStackRun(dims, n_layers, t, [layout], seg_len, seg_p, [rt], inputs, "cuda")
        run.build_caches()
        for _ in range(args.warmup):
            run.forward()
        torch.cuda.synchronize()
        ev = []
        for _ in range(args.steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            run.forward()
            b.record()
            ev.append((a, b))
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        points.append({"config": name, "threshold_layers": t, "ratio": f"{rt[0]}%",
                       "active_rows": int(run.n_act), "ms_per_pass": round(ms, 3),
                       "prefill_tokens_per_s": round(T / (ms * 1e-3), 1)})
        print(f"# {name}: {ms:.3f} ms", file=sys.stderr, flush=True)
        del run, inputs
        torch.cuda.empty_cache()
    full_ms = points[0]["ms_per_pass"]
    for p in points:
        p["speedup_vs_full_recompute"] = round(full_ms / p["ms_per_pass"], 2)
    out = {
        "metric": "chat32k prefill time per 32-layer pass vs full+sparse threshold",
        "unit": "ms", "higher_is_better": False, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": ("chat32k: 32-layer Llama-3-8B-shaped attention stack, "
                                f"120-token instruction + {n_cache}-token reused history + "
                                f"{T - 120 - n_cache - 80}-token uncached last block + 80-token "
                                f"question = {T} tokens"), "tokens": T},
        "points": points,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.sweep:
        sweep(args)
        return
    from segment_level_kv_amd import synth
    from segment_level_kv_amd.stack import HybridStackRun, phase_counts, phase_ms

    qwen = args.workload == "qwen128k"
    agent = args.workload == "agent64k"
    llama1l = args.workload == "llama1l"
    ratios = None
    if llama1l:
        # each segment cached alone at an offset in [0, 8192 - 512]
        dims = synth.LLAMA8B
        seg_lengths = [512] * 8
        layouts = [[("reuse", i) for i in range(8)] + [("new", 256)]]
        ratios = [(15, 100)]
        rng = np.random.default_rng(1022)
        p_src = [int(rng.integers(0, 8192 - 512 + 1)) for _ in seg_lengths]
        n_layers = args.layers if args.layers is not None else 1
        t = args.threshold if args.threshold is not None else 0
        seed = 1002
    elif agent:
        # each pool segment cached alone at an offset in [0, 8192 - L]
        dims = synth.LLAMA8B
        seg_lengths, layouts, ratios = synth.agent_layout()
        rng = np.random.default_rng(1021)
        p_src = [int(rng.integers(0, 8192 - n + 1)) for n in seg_lengths]
        n_layers = args.layers if args.layers is not None else 1
        t = args.threshold if args.threshold is not None else 0
        seed = 1004
    elif qwen:
        # the 32 segments were cached together in a first request, in a seeded
        # order; the measured request reuses them in index order + 1,024 new
        dims = synth.QWEN7B
        seg_lengths, layout = synth.qwen_layout()
        order = np.random.default_rng(1005).permutation(len(seg_lengths))
        p_src = [int(order[i]) * seg_lengths[i] for i in range(len(seg_lengths))]
        n_layers = args.layers if args.layers is not None else 28
        t = args.threshold if args.threshold is not None else 8
        seed = 1005
    else:
        dims = synth.LLAMA8B
        seg_lengths, layout, p_src = synth.rag_layout()
        n_layers = args.layers if args.layers is not None else 32
        t = args.threshold if args.threshold is not None else 4
        seed = 1003
    if not (agent or llama1l):
        layouts, ratios = [layout], [(10, 100)]
    seg_len = {i: n for i, n in enumerate(seg_lengths)}
    seg_p = {i: p for i, p in enumerate(p_src)}
    n_tok = sum(seg_len[v] if k == "reuse" else v for lay in layouts for k, v in lay)
    n_cache = sum(seg_lengths)
    dev = "cuda"
    inputs = synth.TorchStackInputs(seed, dims, n_layers, n_tok, n_cache, t, dev)
    run = HybridStackRun(dims, n_layers, t, layouts, seg_len, seg_p, ratios, inputs, dev)
    run.build_caches()
    torch.cuda.synchronize()
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        run.forward()
    torch.cuda.synchronize()

    timer = {}
    step_ev = []
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for _ in range(args.steps):
        a = torch.cuda.Event(enable_timing=True)
        a.record()
        marks = {}
        run.forward(timer, pipelined=args.pipelined, marks=marks)
        step_ev.append((a, marks["sparse"], marks["end"]))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    ms_step = float(np.mean([a.elapsed_time(e) for a, _, e in step_ev]))
    sparse_wall_ms = float(np.mean([s_.elapsed_time(e) for _, s_, e in step_ev]))
    ph = phase_ms(timer)
    cnt = phase_counts(timer)
    K = args.steps
    n_sparse = n_layers - t
    T = run.n_tok
    # headline: wall time of the selection and the sparse layers (launch
    # stream events around the whole section) per sparse layer
    t_layer_ms = sparse_wall_ms / n_sparse
    value = T / (t_layer_ms * 1e-3)
    phase_sum_ms = (ph.get("realign", 0) + ph.get("recompute", 0) + ph.get("recompute_realign", 0)
                    + ph.get("sparse_attn", 0) + ph.get("select", 0) + ph.get("attn_plan", 0)) / K / n_sparse

    # sparse attention roofline: unmasked MACs of QK^T and PV
    act = run.act_rows[:run.n_act].cpu().numpy().astype(np.int64)
    seq_h = np.asarray(run.seq_start_h, dtype=np.int64)
    pos = act - seq_h[np.searchsorted(seq_h, act, side="right") - 1]     # index in its request
    flops = 4.0 * dims.head_dim * dims.n_q_heads * float(np.sum(pos + 1))
    attn_ms = ph["sparse_attn"] / cnt["sparse_attn"]
    achieved = flops / (attn_ms * 1e-3) / 1e12
    # the committed counters are of the rag32k workload
    traffic = None if (qwen or agent or llama1l) else measured_traffic()
    # other phases (per launch)
    reused = sum(seg_len[v] for lay in layouts for k, v in lay if k == "reuse")
    realign_bytes = 2.0 * reused * dims.n_kv_heads * dims.head_dim * 2 * 2   # K+V read + write
    realign_ms = ph["realign"] / cnt["realign"]
    rec_flops = 2.0 * run.n_act * dims.qkv_rows * dims.hidden
    rec_ms = ph["recompute"] / cnt["recompute"]
    full_rec_ms = ph.get("full_recompute", 0) / max(cnt.get("full_recompute", 1), 1)
    full_attn_ms = ph.get("full_attn", 0) / max(cnt.get("full_attn", 1), 1)
    full_attn_flops = 4.0 * dims.head_dim * dims.n_q_heads * (T * (T + 1) / 2)
    sel_ms = ph.get("select", 0) / max(cnt.get("select", 1), 1)
    # layer l's recompute launch carrying layer l+1's realign (all sparse
    # layers but the last); "realign" and "recompute" above are the first
    # layer's realign and the last layer's recompute, each alone
    rr_ms = ph.get("recompute_realign", 0) / max(cnt.get("recompute_realign", 1), 1)
    plan_ms = ph.get("attn_plan", 0) / max(cnt.get("attn_plan", 1), 1)

    out = {
        "metric": METRIC_QWEN if qwen else (METRIC_AGENT if agent else (METRIC_1L if llama1l else METRIC)),
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"llama1l: {n_layers}-layer Llama-3-8B-shaped attention stack, 8 reused 512-token "
                         f"segments (each cached alone at an offset in [0, 7680]) + 256 new = {T} tokens, "
                         "ratio 15%, selection inside layer 0") if llama1l else
                        (f"agent64k: {n_layers}-layer Llama-3-8B-shaped attention stack, {len(layouts)} "
                         f"requests ({T} tokens) drawn from a pool of 64 reused segments of 32-2048 tokens, "
                         "no new tokens (tail fallback), ratios 5-30% per request, selection inside "
                         "layer 0") if agent else
                        (f"qwen128k: {n_layers}-layer Qwen2.5-7B-shaped attention stack (hidden 3584, "
                         "28/4 heads, head_dim 128), 32 reused 4000-token segments (cached together in a "
                         f"seeded order) + 1024 new = {T} tokens, full layers 0-{t - 1}, sparse "
                         f"{t}-{n_layers - 1}, ratio 10%") if qwen else
                        ("rag32k: 32-layer Llama-3-8B-shaped attention stack (hidden 4096, 32/8 heads, "
                         "head_dim 128), 512 reused system + 16x1920 reused passages + 256 new "
                         f"= {T} tokens, full layers 0-{t - 1}, sparse {t}-{n_layers - 1}, ratio 10%"),
            "tokens": T, "active_rows": int(run.n_act), "selected": int(run.n_sel),
            "sparse_q_rows": int(run.n_sq), "layers": n_layers, "threshold": t, "page_size": 16,
            "streams": 2 if args.pipelined else 1,
        },
        "attn_pct_mfma_bf16_peak": round(100.0 * achieved / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "kernel": ("sx_sparse_attn_run (attn_fwd<true>; attn_merge only when tiles are split), one "
                       "launch per sparse layer over the work list sx_sparse_attn_plan builds once per pass"),
            "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "flops_per_launch": flops, "avg_launch_ms": round(attn_ms, 4),
        },
        "phases_ms_per_launch": {
            "realign": round(realign_ms, 4), "recompute_active": round(rec_ms, 4),
            "recompute_active_with_next_realign": round(rr_ms, 4),
            "sparse_attn": round(attn_ms, 4), "select": round(sel_ms, 4), "attn_plan": round(plan_ms, 4),
            "full_recompute": round(full_rec_ms, 4), "full_attn": round(full_attn_ms, 4),
        },
        "phases_rate": {
            "realign_GBps": round(realign_bytes / (realign_ms * 1e-3) / 1e9, 1),
            "recompute_active_TFLOPs": round(rec_flops / (rec_ms * 1e-3) / 1e12, 1),
            "full_attn_TFLOPs": round(full_attn_flops / (full_attn_ms * 1e-3) / 1e12, 1) if full_attn_ms else None,
            "full_recompute_TFLOPs": round(2.0 * T * dims.qkv_rows * dims.hidden / (full_rec_ms * 1e-3) / 1e12, 1) if full_rec_ms else None,
        },
        "full_stack_tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "sparse_layer_ms": round(t_layer_ms, 4),
        "sparse_layer_ms_phase_sum": round(phase_sum_ms, 4),
        "pipelined": bool(args.pipelined),
        "full_layer_ms": round(full_rec_ms + full_attn_ms, 4),
        "wall_s_timed": round(wall, 3),
    }
    # every kernel of the sparse layer (and the full layer) against its roofline,
    # per launch; the selection's work is the QK^T of the Sparse-Q rows over
    # their key prefixes for the scores, plus the same again for the LSE probe
    # when the selection runs inside layer 0 (t = 0; at a boundary t > 0 the
    # LSE comes from layer t-1's full attention)
    sq_tok = np.asarray(run.plan["sq_rows"], dtype=np.int64)
    sq = sq_tok - seq_h[np.searchsorted(seq_h, sq_tok, side="right") - 1]
    sel_flops = (2 if t == 0 else 1) * (2.0 * dims.head_dim * dims.n_q_heads * float(np.sum(sq + 1)))
    full_rec_flops = 2.0 * T * dims.qkv_rows * dims.hidden
    rate = lambda work, ms, unit: round(work / (ms * 1e-3) / unit, 1) if ms else None
    out["kernels"] = {
        "realign": {"GB/s": rate(realign_bytes, realign_ms, 1e9), "peak": PEAK_HBM_GBS,
                    "frac": round(realign_bytes / (realign_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "recompute_active": {"TFLOP/s": rate(rec_flops, rec_ms, 1e12), "peak": PEAK_BF16_TFLOPS,
                             "frac": round(rec_flops / (rec_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "sparse_attn": {"TFLOP/s": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                        "frac": round(achieved / PEAK_BF16_TFLOPS, 4)},
        "select": {"TFLOP/s": rate(sel_flops, sel_ms, 1e12), "peak": PEAK_BF16_TFLOPS,
                   "frac": round(sel_flops / (sel_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4) if sel_ms else None},
        "full_recompute": {"TFLOP/s": rate(full_rec_flops, full_rec_ms, 1e12), "peak": PEAK_BF16_TFLOPS,
                           "frac": round(full_rec_flops / (full_rec_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4) if full_rec_ms else None},
        "full_attn": {"TFLOP/s": rate(full_attn_flops, full_attn_ms, 1e12), "peak": PEAK_BF16_TFLOPS,
                      "frac": round(full_attn_flops / (full_attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4) if full_attn_ms else None},
    }
    out["active_rows_per_s_per_layer"] = round(run.n_act / (t_layer_ms * 1e-3), 1)
    if full_rec_ms and full_attn_ms:
        out["speedup_vs_full_layer"] = round((full_rec_ms + full_attn_ms) / t_layer_ms, 2)
    out["decode_attn"] = decode_measure(run, dims, n_layers, t)
    peak = mfma_peak_measure()
    out["mfma_peak_measured"] = peak
    out["attn_pct_measured_mfma_peak"] = round(100.0 * achieved / peak["TFLOP/s"], 2)
    out["attn_pct_measured_mfma_peak_random_operands"] = round(
        100.0 * achieved / peak["random_operands_TFLOP/s"], 2)
    if not args.no_cpu_baseline and not (qwen or agent or llama1l):
        out["cpu_baseline"] = cpu_baseline(dims, run.plan, n_sparse, T, reused)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
