"""sx_decode_attn_noalloc against sx_decode_attn (GPU).

The no-allocation entry point runs the same decode kernels with their
partial results in a static scratch array instead of a caller workspace, so
its outputs must equal sx_decode_attn's bit for bit.  Two calls in a row, the
second with a smaller batch (the scratch keeps the first call's contents),
and a batch whose workspace need exceeds the scratch (rejected before any
launch).  The smaller call is also checked against the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from segment_level_kv_amd import _lib as L
from segment_level_kv_amd import layer as LY
from segment_level_kv_amd import synth
from tests.gpu_util import assert_close_bf16, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
LLAMA = synth.Dims(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, theta=5e5, dtype="bf16")


def _inputs(dims, lens, seed):
    rng = np.random.default_rng(seed)
    seq = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    req_pages = [(n + 15) // 16 for n in lens]
    n_pages = sum(req_pages) + 2
    hkv, d = dims.n_kv_heads, dims.head_dim
    k = synth.to_storage(rng.standard_normal((n_pages, hkv, 16, d)), "bf16")
    v = synth.to_storage(rng.standard_normal((n_pages, hkv, d, 16)), "bf16")
    perm = rng.permutation(n_pages).astype(np.int32)
    bt = np.full((len(lens), max(max(req_pages), 1)), -1, np.int32)
    o = 0
    for r, n in enumerate(req_pages):
        bt[r, :n] = perm[o:o + n]
        o += n
    q = synth.to_storage(rng.standard_normal((len(lens), dims.n_q_heads, d)), "bf16")
    pool = LY.PagePool(torch.from_numpy(k).to(torch.bfloat16).to(DEV),
                       torch.from_numpy(v).to(torch.bfloat16).to(DEV))
    lay = LY.DeviceLayout(seq, bt, LY.rope_table(dims.theta, d, 16, DEV), DEV)
    return seq, bt, k, v, q, pool, lay


def _both(dims, lens, seed):
    seq, bt, kh, vh, qh, pool, lay = _inputs(dims, lens, seed)
    n_req = len(lens)
    cd = LY.make_dims(dims)
    q = torch.from_numpy(qh).to(torch.bfloat16).to(DEV)
    outs = []
    for noalloc in (False, True):
        o = torch.full((n_req, dims.n_q_heads * dims.head_dim), 3.0, dtype=torch.bfloat16, device=DEV)
        lse = torch.zeros((n_req, dims.n_q_heads), dtype=torch.float32, device=DEV)
        if noalloc:
            L.sx_decode_attn_noalloc(cd, lay.struct, q, pool.struct(), o, lse)
        else:
            ws = LY.workspace(L.SX_OP_DECODE, cd, int(seq[-1]), 0, n_req, DEV)
            L.sx_decode_attn(cd, lay.struct, q, pool.struct(), o, lse, ws)
        torch.cuda.synchronize()
        outs.append((o, lse))
    (o_ws, l_ws), (o_na, l_na) = outs
    assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16)), "O differs from sx_decode_attn"
    assert torch.equal(l_ws.view(torch.int32), l_na.view(torch.int32)), "LSE differs from sx_decode_attn"
    return seq, bt, kh, vh, qh, o_na.float().cpu().double().numpy()


def test_noalloc_decode_equals_workspace_call():
    """A larger batch, then a smaller one on the same scratch."""
    say("[noalloc] call 1: lens [31745, 2000, 700]")
    _both(LLAMA, [31745, 2000, 700], seed=41)
    say("[noalloc] call 2: lens [129, 17]")
    seq, bt, kh, vh, qh, og = _both(LLAMA, [129, 17], seed=42)
    for r, T in enumerate([129, 17]):
        idx = np.arange(T)
        K = kh[bt[r][idx // 16], :, idx % 16, :]
        V = vh[bt[r][idx // 16], :, :, idx % 16]
        ref, _ = oracle.causal_attention(qh[r:r + 1], np.array([T - 1]), K, V)
        assert_close_bf16(og[r:r + 1], ref.reshape(1, -1), what=f"noalloc decode request {r}")


def test_noalloc_decode_rejects_batch_beyond_scratch():
    """300 Llama-shaped requests need about 5 MB of partials: SX_EWORKSPACE,
    nothing launched, outputs untouched."""
    lens = [1] * 300
    seq, bt, kh, vh, qh, pool, lay = _inputs(LLAMA, lens, seed=43)
    cd = LY.make_dims(LLAMA)
    need = L.sx_workspace_bytes(L.SX_OP_DECODE, cd, int(seq[-1]), 0, len(lens))
    assert need > (4 << 20)
    q = torch.from_numpy(qh).to(torch.bfloat16).to(DEV)
    o = torch.full((len(lens), LLAMA.n_q_heads * LLAMA.head_dim), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(L.SxError) as e:
        L.sx_decode_attn_noalloc(cd, lay.struct, q, pool.struct(), o, None)
    assert e.value.status == L.SX_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())
