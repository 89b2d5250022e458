"""GPU parity of the full+sparse hybrid stack (§3.4) against the oracle.

A 3-layer bf16 stack over one chat-shaped request (instruction | reused
history segment | new run | reused segment | the history's last partial
block | question), for every threshold t in {0, 1, 2}:
  - layers < t are full layers: every row recomputed and attending;
  - the selection uses layer t-1's probabilities (its Q of the Sparse-Q
    rows, its fresh K and its LSE), or, for t = 0, the probe inside layer 0
    over its mixed cache;
  - layers >= t realign, recompute A = I_nr U S and attend.
Each layer takes its own seeded inputs (layer input rows, weights and the
rows the segment caches were built from), read back from the device for
the oracle.  Compared: every full layer's O; the selection as in the
single-layer test (exactly the top-k of the GPU's scores; the GPU's scores
within 1e-5 * max s of the oracle's scores from the GPU's stored queries,
keys and, at the boundary, the oracle's LSE of them; the oracle's top-k up
to the near-tie band), with the boundary LSE of sx_full_attn checked too;
and every sparse layer's O over the rows both active sets share.
"""

import numpy as np
import pytest
import torch

import oracle
from segment_level_kv_amd import synth
from segment_level_kv_amd.layer import gather_logical
from segment_level_kv_amd.stack import HybridStackRun
from tests.gpu_util import (assert_o_bf16, check_selection, probe_lse_and_scores, say,
                            selection_contract)

pytestmark = pytest.mark.gpu
DEV = "cuda"

SMALL = synth.Dims(hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=128, theta=5e5, dtype="bf16")
LAYOUT = [("new", 40), ("reuse", 0), ("new", 24), ("reuse", 1), ("new", 9), ("new", 30)]
SEG_LEN = {0: 304, 1: 192}
SEG_P = {0: 0, 1: 700}
RATIO = (20, 100)
N_LAYERS = 3


def _host(t):
    return t.float().cpu().double().numpy()


def _split(w, d):
    hq, hkv, hd = d.n_q_heads, d.n_kv_heads, d.head_dim
    return w[:hq * hd], w[hq * hd:(hq + hkv) * hd], w[(hq + hkv) * hd:]


def _segments(xc, wq, wk, wv, d):
    """Oracle caches: each segment projected alone at its original positions."""
    out, off, dst = [], {}, 0
    o = 0
    for s in sorted(SEG_LEN):
        off[s] = o
        o += SEG_LEN[s]
    for kind, v in LAYOUT:
        if kind == "reuse":
            rows = xc[off[v]:off[v] + SEG_LEN[v]]
            pos = np.arange(SEG_LEN[v]) + SEG_P[v]
            _, k, vv = oracle.project_rows(rows, wq, wk, wv, pos, d.theta, d.n_q_heads,
                                           d.n_kv_heads, d.head_dim, d.dtype, want_q=False)
            out.append((dst, SEG_P[v], k, vv))
            dst += SEG_LEN[v]
        else:
            dst += v
    return out


@pytest.mark.parametrize("t,pipelined", [(0, False), (1, False), (2, False), (0, True), (1, True)])
def test_hybrid_stack_parity(t, pipelined):
    """pipelined: the sparse layers on two streams (layer l+1's realign and
    recompute while layer l attends); the results must not change."""
    d = SMALL
    say(f"[stack] layers={N_LAYERS} threshold={t} pipelined={pipelined}")
    n_tok = sum(SEG_LEN[v] if k == "reuse" else v for k, v in LAYOUT)
    n_cache = sum(SEG_LEN.values())
    inputs = synth.TorchStackInputs(77 + t, d, N_LAYERS, n_tok, n_cache, t, DEV)
    run = HybridStackRun(d, N_LAYERS, t, [LAYOUT], SEG_LEN, SEG_P, [RATIO], inputs, DEV,
                         keep_probe_cache=True)
    run.build_caches()
    run.forward(keep_full_outputs=True, pipelined=pipelined)
    torch.cuda.synchronize()

    pieces = [(k, SEG_LEN[v] if k == "reuse" else v) for k, v in LAYOUT]
    plan = oracle.plan_request(pieces, RATIO)
    sq, k = plan["sq"], plan["k"]
    sel = np.sort(run.sel_rows[:run.n_sel].cpu().numpy().astype(np.int64))
    act = run.act_rows[:run.n_act].cpu().numpy().astype(np.int64)
    assert run.n_sel == k and np.array_equal(act, np.union1d(sq, sel))

    T = n_tok
    s_gpu = run.scores.cpu().double().numpy()
    q_sq_gpu = _host(run.q_full[:run.n_sq]) if t == 0 else _host(run.q_full)[sq]
    if t == 0:
        k_probe, _ = gather_logical(type(run.req_pools[0])(run.probe_k, run.req_pools[0].v),
                                    run.block_table[0], T)
    else:
        k_probe, _ = gather_logical(run.req_pools[t - 1], run.block_table[0], T)
    lse_g, s_from_gpu = probe_lse_and_scores(q_sq_gpu, sq, k_probe)
    nd, serr = check_selection(s_gpu, sel, s_from_gpu, plan["cand"], k, what=f"threshold {t}")
    say(f"  selection from the GPU's stored values: score err/max={serr:.2e} differences={nd}")
    if t > 0:   # the boundary LSE that sx_full_attn returned for the Sparse-Q rows
        lse_gpu = run.lse_full.cpu().double().numpy()[sq]
        lerr = float(np.max(np.abs(lse_gpu - lse_g)))
        assert lerr <= 1e-4, f"boundary LSE error {lerr:.3g}"
        say(f"  boundary LSE max abs err={lerr:.2e}")

    S_ref = None
    for l in range(t):
        x, w, _ = inputs(l)
        wq, wk, wv = _split(_host(w), d)
        ref = oracle.full_layer(_host(x), wq, wk, wv, d.theta, d.n_q_heads, d.n_kv_heads,
                                d.head_dim, d.dtype)
        oerr = assert_o_bf16(_host(run.o_full_layers[l]), ref["O_exact"], what=f"full layer {l}")
        say(f"  full layer {l}: O max abs err={oerr:.3g}")
        if l == t - 1:   # boundary: probabilities of layer t-1 (§3.4)
            scores = oracle.attention_mass_scores(ref["q"][sq], sq, ref["K"], ref["lse"][sq])
            tol = 1e-4 * scores.max() + 2e-3 * scores.max()
            nd = selection_contract(sel, scores, plan["cand"], k, tol)
            say(f"  boundary selection: k={k} differences={nd}")
            S_ref = oracle.select_topk(scores, plan["cand"], k)

    for l in range(t, N_LAYERS):
        x, w, xc = inputs(l)
        wq, wk, wv = _split(_host(w), d)
        segs = _segments(_host(xc), wq, wk, wv, d)
        out = oracle.sparse_layer(_host(x), wq, wk, wv, plan, segs, d.theta, d.n_q_heads,
                                  d.n_kv_heads, d.head_dim, d.dtype, selected=S_ref)
        if S_ref is None:   # t == 0: the probe of layer 0 selects
            tol = 1e-4 * out["scores"].max() + 2e-3 * out["scores"].max()
            nd = selection_contract(sel, out["scores"], plan["cand"], k, tol)
            say(f"  in-layer selection: k={k} differences={nd}")
            S_ref = out["S"]
        common, gi, ri = np.intersect1d(act, out["A"], return_indices=True)
        assert len(common) >= len(sq)
        oerr = assert_o_bf16(_host(run.o_act[l])[gi], out["O_exact"][ri], what=f"sparse layer {l}")
        say(f"  sparse layer {l}: O max abs err={oerr:.3g}")
