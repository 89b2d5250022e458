"""Run-to-run determinism of the GPU path (GPU).

Every reduction runs in a fixed order and no floating-point atomics are
used, so running the same call twice must give the same bits: the Llama
layer (scores, selection, active set, O, LSE and the whole page pools), and
the sparse attention at the rag32k shape (3,379 active rows over 31,488
tokens: tiles never split) and with few rows (tiles split into key chunks
and merged).
"""

import numpy as np
import pytest
import torch

from segment_level_kv_amd import _lib as L
from segment_level_kv_amd import layer as LY
from segment_level_kv_amd import synth
from segment_level_kv_amd.layer import SparseXLayerRun
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _same(a, b, what):
    a = a.contiguous().view(torch.uint8)
    b = b.contiguous().view(torch.uint8)
    assert torch.equal(a, b), f"{what} differs between two runs"


def test_layer_runs_are_bit_identical():
    case = synth.llama_layer_case()
    say("[determinism] llama layer, two runs")
    runs = []
    for _ in range(2):
        run = SparseXLayerRun(case).run()
        torch.cuda.synchronize()
        runs.append(run)
    a, b = runs
    for name in ("scores", "sel_rows", "act_rows", "o", "lse", "q_sq", "q_act"):
        _same(getattr(a, name), getattr(b, name), name)
    _same(a.pool.k, b.pool.k, "K pool")
    _same(a.pool.v, b.pool.v, "V pool")


def _attention_twice(n_sel, seed):
    d = synth.LLAMA8B
    T = 31488
    rng = np.random.default_rng(seed)
    n_pages = (T + 15) // 16 + 8
    perm = rng.permutation(n_pages).astype(np.int32)
    bt = perm[:(T + 15) // 16][None, :].copy()
    rows = np.union1d(np.arange(T - 256, T), rng.choice(T - 256, size=n_sel, replace=False)).astype(np.int32)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    pool = LY.PagePool.alloc(n_pages, d, DEV, fill_guard=False)
    pool.k.copy_(torch.randn(pool.k.shape, generator=g, device=DEV).to(torch.bfloat16))
    pool.v.copy_(torch.randn(pool.v.shape, generator=g, device=DEV).to(torch.bfloat16))
    q = torch.randn((len(rows), d.n_q_heads, d.head_dim), generator=g, device=DEV).to(torch.bfloat16)
    lay = LY.DeviceLayout(np.array([0, T], np.int32), bt, LY.rope_table(d.theta, d.head_dim, 16, DEV), DEV)
    cd = LY.make_dims(d)
    rt = torch.from_numpy(rows).to(DEV)
    rs = torch.tensor([0, len(rows)], dtype=torch.int32, device=DEV)
    ws = LY.workspace(L.SX_OP_SPARSE_ATTN, cd, T, len(rows), 1, DEV)
    outs = []
    for _ in range(2):
        o = torch.empty((len(rows), d.n_q_heads * d.head_dim), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((len(rows), d.n_q_heads), dtype=torch.float32, device=DEV)
        L.sx_sparse_attn(cd, lay.struct, q, rt, rs, len(rows), pool.struct(), o, lse, ws)
        torch.cuda.synchronize()
        outs.append((o, lse))
    _same(outs[0][0], outs[1][0], "O")
    _same(outs[0][1], outs[1][1], "LSE")


@pytest.mark.parametrize("n_sel,what", [(3123, "rag32k active set, no split"),
                                        (100, "few rows, split tiles")])
def test_sparse_attention_runs_are_bit_identical(n_sel, what):
    say(f"[determinism] sparse attention at 32K: {what}")
    _attention_twice(n_sel, seed=n_sel)
