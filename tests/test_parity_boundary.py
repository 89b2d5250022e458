"""GPU parity of the boundary selection at full size (SparseX paper §3.4:
at the boundary layer one Sparse-Q estimation uses the Sparse-Q rows and the
K/V of the last full-attention layer; §3.2 aggregated score; §3.3 top-k).

The hybrid stack runs layers 0 .. t-1 as full layers on the GPU, then the
selection from layer t-1's probabilities: the log-sum-exp that sx_full_attn
returned for the Sparse-Q rows, their queries read through q_index from the
full layer's Q buffer, and the per-kv-head score grid -- the launch shapes the
benchmark times.  Then at least one sparse layer.  Compared with the oracle:
  - layer t-1's keys of every token and the Sparse-Q queries, against the
    oracle's projection of that layer's input (bf16 storage tolerance);
  - the boundary LSE against the oracle's LSE from the GPU's stored queries
    and keys (1e-4 in natural-log units);
  - the scores against the oracle's scores from those same stored values
    (1e-5 * max s), and the selection: exactly the top-k of the GPU's scores,
    and the oracle's top-k up to the near-tie band;
  - sampled output rows of the last full layer (max |g - r| <= 1e-2 where
    |r| < 2.56) against the oracle's attention over the stored Q, K, V;
  - rag32k also: sampled rows of the first sparse layer, from the oracle's own
    layer with the GPU's selection.
Inputs are generated on the device (seeded) and read back for the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from segment_level_kv_amd import synth
from segment_level_kv_amd.layer import gather_logical
from segment_level_kv_amd.stack import HybridStackRun
from tests.gpu_util import (assert_close_bf16, assert_o_bf16, check_selection,
                            probe_lse_and_scores, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _host(t):
    return t.float().cpu().double().numpy()


def _split(w, d):
    hq, hkv, hd = d.n_q_heads, d.n_kv_heads, d.head_dim
    return w[:hq * hd], w[hq * hd:(hq + hkv) * hd], w[(hq + hkv) * hd:]


def _run(d, seg_lengths, layout, p_src, ratio, t, seed):
    seg_len = {i: n for i, n in enumerate(seg_lengths)}
    seg_p = {i: p for i, p in enumerate(p_src)}
    n_tok = sum(seg_len[v] if k == "reuse" else v for k, v in layout)
    n_cache = sum(seg_lengths)
    n_layers = t + 1
    say(f"[boundary] {n_tok} tokens, full layers 0-{t - 1}, selection at {t - 1}, sparse layer {t}")
    inputs = synth.TorchStackInputs(seed, d, n_layers, n_tok, n_cache, t, DEV)
    run = HybridStackRun(d, n_layers, t, [layout], seg_len, seg_p, [ratio], inputs, DEV)
    run.build_caches()
    run.forward()
    torch.cuda.synchronize()
    pieces = [(k, seg_len[v] if k == "reuse" else v) for k, v in layout]
    plan = oracle.plan_request(pieces, ratio)
    return run, inputs, plan, seg_len, seg_p, n_tok


def _check_boundary(d, run, inputs, plan, n_tok, t, n_out_rows):
    sq, k, cand = plan["sq"], plan["k"], plan["cand"]
    T = n_tok
    sel = np.sort(run.sel_rows[:run.n_sel].cpu().numpy().astype(np.int64))
    act = run.act_rows[:run.n_act].cpu().numpy().astype(np.int64)
    assert run.n_sel == k and np.array_equal(act, np.union1d(sq, sel))
    l = t - 1
    x, w, _ = inputs(l)
    wq, wk, wv = _split(_host(w), d)
    K_g, V_g = gather_logical(run.req_pools[l], run.block_table[0], T)
    q_sq_g = _host(run.q_full[torch.as_tensor(sq, device=DEV)])
    say(f"[boundary] oracle projection of layer {l}")
    xh = _host(x)
    q_ref, k_ref, v_ref = oracle.project_rows(xh, wq, wk, wv, np.arange(T), d.theta, d.n_q_heads,
                                              d.n_kv_heads, d.head_dim, d.dtype, want_q=False)
    assert_close_bf16(K_g, k_ref, what=f"layer {l} keys")
    assert_close_bf16(V_g, v_ref, what=f"layer {l} values")
    q_ref, _, _ = oracle.project_rows(xh[sq], wq, wk, wv, sq, d.theta, d.n_q_heads, d.n_kv_heads,
                                      d.head_dim, d.dtype)
    assert_close_bf16(q_sq_g, q_ref, what="Sparse-Q queries")
    del xh, k_ref, v_ref
    say("[boundary] oracle LSE and scores from the GPU's stored queries and keys")
    lse_ref, s_ref = probe_lse_and_scores(q_sq_g, sq, K_g)
    lse_g = run.lse_full.cpu().double().numpy()[sq]
    lerr = float(np.max(np.abs(lse_g - lse_ref)))
    assert lerr <= 1e-4, f"boundary LSE max abs err {lerr:.3g}"
    s_g = run.scores.cpu().double().numpy()
    nd, serr = check_selection(s_g, sel, s_ref, cand, k, what="boundary")
    # sampled output rows of the full layer, over the stored Q, K, V
    rows = np.unique(np.concatenate([np.linspace(0, T - 1, n_out_rows).round().astype(np.int64),
                                     sq[:: max(1, len(sq) // 8)]]))
    q_rows = _host(run.q_full[torch.as_tensor(rows, device=DEV)])
    o_ref, _ = oracle.causal_attention(q_rows, rows, K_g, V_g)
    o_g = _host(run.o_full[torch.as_tensor(rows, device=DEV)])
    oerr = assert_o_bf16(o_g, o_ref.reshape(len(rows), -1), what=f"full layer {l} sampled O")
    say(f"[boundary] k={k} LSE max abs err={lerr:.2e} score err/max={serr:.2e} "
        f"selection differences={nd} full-layer O max abs err={oerr:.3g} ({len(rows)} rows)")
    return sel


def test_rag32k_boundary_selection_full_size():
    """rag32k: 31,488 tokens, Llama-3-8B dims, threshold 4 (the bench's
    configuration), selection at layer 3, then sparse layer 4."""
    d = synth.LLAMA8B
    seg_lengths, layout, p_src = synth.rag_layout()
    t = 4
    run, inputs, plan, seg_len, seg_p, n_tok = _run(d, seg_lengths, layout, p_src, (10, 100), t,
                                                    seed=2003)
    sel = _check_boundary(d, run, inputs, plan, n_tok, t, n_out_rows=24)
    # first sparse layer, sampled rows, with the GPU's selection
    x, w, xc = inputs(t)
    wq, wk, wv = _split(_host(w), d)
    xch = _host(xc)
    segs, off, dst = [], 0, 0
    starts = {}
    for s in sorted(seg_len):
        starts[s] = off
        off += seg_len[s]
    say(f"[boundary] oracle sparse layer {t} (segment caches, selected rows, sampled attention)")
    for kind, v in layout:
        if kind == "reuse":
            pos = np.arange(seg_len[v]) + seg_p[v]
            _, kc, vc = oracle.project_rows(xch[starts[v]:starts[v] + seg_len[v]], wq, wk, wv, pos,
                                            d.theta, d.n_q_heads, d.n_kv_heads, d.head_dim,
                                            d.dtype, want_q=False)
            segs.append((dst, seg_p[v], kc, vc))
            dst += seg_len[v]
        else:
            dst += v
    del xch
    out = oracle.sparse_layer(_host(x), wq, wk, wv, plan, segs, d.theta, d.n_q_heads,
                              d.n_kv_heads, d.head_dim, d.dtype, selected=sel, out_rows=24)
    act = run.act_rows[:run.n_act].cpu().numpy().astype(np.int64)
    common, gi, ri = np.intersect1d(act, out["O_rows"], return_indices=True)
    assert len(common) == len(out["O_rows"])
    o_g = _host(run.o_act[t])[gi]
    oerr = assert_o_bf16(o_g, out["O_exact"][ri], what=f"sparse layer {t} sampled O")
    say(f"[boundary] sparse layer {t}: O max abs err={oerr:.3g} ({len(common)} rows)")


def test_qwen128k_boundary_selection_full_size():
    """qwen128k: 129,024 tokens, Qwen2.5-7B dims (28 q / 4 kv heads),
    threshold 8, selection at layer 7."""
    d = synth.QWEN7B
    seg_lengths, layout = synth.qwen_layout()
    rng = np.random.default_rng(2005)
    p_src = [int(v) for v in rng.integers(0, 128 * 1024 - seg_lengths[0], len(seg_lengths))]
    run, inputs, plan, _, _, n_tok = _run(d, seg_lengths, layout, p_src, (10, 100), 8, seed=2005)
    _check_boundary(d, run, inputs, plan, n_tok, 8, n_out_rows=12)
