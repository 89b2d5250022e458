"""GPU parity at the full sizes of the workloads (sampled outputs).

One sparse layer of each large configuration at its real shape, with the
selection inside the layer, through the same entry points and launch shapes
the bench times (realign, recompute of the active rows, sparse attention):
  - rag32k: Llama-3-8B dims, 31,488 tokens (a 512-token system segment and
    16 passages of 1,920 tokens, reused, then a 256-token query), ratio 10%;
  - agent batch: 4 requests of about 64K tokens each drawn from a shared
    pool of 64 segments (log-uniform lengths in [32, 2048]), no new tokens
    (the tail fallback supplies the Sparse-Q rows), ratios 5-30%;
  - qwen128k: Qwen2.5-7B dims (28 q / 4 kv heads), 32 reused segments of
    4,000 tokens and a 1,024-token suffix (129,024 tokens), ratio 10%.
The oracle computes each request's whole layer itself: every segment cache,
the realignment, the Sparse-Q probe over all keys, the scores and the top-k;
only the final attention is sampled (rows spread evenly over A).  Compared:
every score (against the oracle's scores from the GPU's stored queries and
probe-time keys, to 1e-5 * max s, and end to end within the bf16 rounding
band), the selection (exactly the top-k of the GPU's scores; the oracle's
top-k up to the near-tie band), the Sparse-Q queries, the final mixed K/V
cache of every token, and the sampled output rows (max |g - r| <= 1e-2 where
|r| < 2.56).
"""

import numpy as np
import pytest
import torch

import oracle
from segment_level_kv_amd import synth
from segment_level_kv_amd.layer import SparseXLayerRun
from tests.gpu_util import (BF16_STEP_REL, assert_close_bf16, assert_close_bf16_rotated,
                            assert_o_bf16, check_selection, probe_lse_and_scores, say)

pytestmark = pytest.mark.gpu


def _check_full_size(case, n_sample):
    d = case.dims
    n_req = len(case.requests)
    say(f"[fullsize] {case.name}: {sum(case.n_tokens(r) for r in range(n_req))} tokens, "
        f"{n_req} request(s); GPU layer")
    run = SparseXLayerRun(case, keep_probe_cache=True).run()
    torch.cuda.synchronize()
    seq = run.plan["seq_start"]
    k_all = run.plan["k"]
    sel = run.sel_rows.cpu().numpy().astype(np.int64)
    act = run.act_rows.cpu().numpy().astype(np.int64)
    scores = run.scores.cpu().double().numpy()
    o_gpu = run.o.float().cpu().double().numpy()
    sel_off = act_off = 0
    for r in range(n_req):
        say(f"[fullsize] oracle, request {r}")
        plan = oracle.plan_request(case.piece_lengths(r), case.requests[r].ratio)
        segs = []
        for dst, sid in case.reuse_runs(r):
            sg = case.segments[sid]
            pos = np.arange(sg.length) + sg.p_src
            _, kc, vc = oracle.project_rows(sg.x_cache, case.wq, case.wk, case.wv, pos, d.theta,
                                            d.n_q_heads, d.n_kv_heads, d.head_dim, d.dtype,
                                            want_q=False)
            segs.append((dst, sg.p_src, kc, vc))
        ref = oracle.sparse_layer(case.request_x(r), case.wq, case.wk, case.wv, plan, segs,
                                  d.theta, d.n_q_heads, d.n_kv_heads, d.head_dim, d.dtype,
                                  out_rows=n_sample)
        T, k = plan["T"], plan["k"]
        assert k == int(k_all[r])
        s_gpu = scores[seq[r]:seq[r] + T]
        s_ref = ref["scores"]
        assert np.all(np.abs(s_gpu - s_ref) <= 2e-3 * s_ref + 1e-4 * s_ref.max()), \
            f"scores: max abs err {np.max(np.abs(s_gpu - s_ref)):.3g}"
        q_g = run.sq_queries(r)
        assert_close_bf16(q_g, ref["q_sq"], what=f"Sparse-Q queries {r}")
        say(f"[fullsize] oracle scores from the GPU's stored values, request {r}")
        _, s_from_gpu = probe_lse_and_scores(q_g, plan["sq"], run.probe_keys(r))
        g_sel = sel[sel_off:sel_off + k] - seq[r]
        nd, serr = check_selection(s_gpu, g_sel, s_from_gpu, plan["cand"], k, what=f"request {r}")
        n_act = len(plan["sq"]) + k
        a_gpu = act[act_off:act_off + n_act] - seq[r]
        assert np.array_equal(a_gpu, np.union1d(plan["sq"], g_sel))
        Kg, Vg = run.request_cache(r)
        same = np.ones(T, dtype=bool)
        same[np.setxor1d(g_sel, ref["S"])] = False
        assert_close_bf16_rotated(Kg[same], ref["K"][same], what=f"K cache {r}")
        assert_close_bf16(Vg[same], ref["V"][same], rel=BF16_STEP_REL, what=f"V cache {r}")
        rows = ref["O_rows"]
        common, gi, ri = np.intersect1d(a_gpu, rows, return_indices=True)
        assert len(common) >= len(rows) - nd
        oerr = assert_o_bf16(o_gpu[act_off + gi], ref["O_exact"][ri], what=f"sampled O rows {r}")
        say(f"[fullsize]   T={T} k={k} score err/max={serr:.2e} selection differences={nd} "
            f"sampled rows={len(common)} O max abs err={oerr:.3g}")
        sel_off += k
        act_off += n_act


def test_rag32k_layer_full_size_sampled():
    _check_full_size(synth.rag32k_case(), 40)


def test_agent_batch_full_size_sampled():
    _check_full_size(synth.agent_case(n_req=4, target=65536), 16)


def test_qwen128k_layer_full_size_sampled():
    _check_full_size(synth.qwen128k_case(), 24)
