"""GPU parity of decode attention over the paged cache (sx_decode_attn).

One query row per request, at its last token, attending to every token of
the request's cache.  The oracle is the causal attention of that single row
(the same function that defines prefill attention).  Cases: ragged request
lengths around the 16-token page and 32-token unit edges, empty requests,
non-power-of-two GQA groups, page tails and unused pages filled with NaN
(masking must keep them out), and full 32K-token requests in the launch
configuration the bench uses.
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

SHAPES = {
    "llama": synth.Dims(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, theta=5e5, dtype="bf16"),
    "qwen": synth.Dims(hidden=3584, n_q_heads=28, n_kv_heads=4, head_dim=128, theta=1e6, dtype="bf16"),
}
NAN_BF16 = 0x7FC0


def _case(dims, lens, seed, qscale=1.0):
    """Random pages, a shuffled block table, NaN in every slot no request owns."""
    rng = np.random.default_rng(seed)
    seq = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    req_pages = [(n + 15) // 16 for n in lens]
    n_pages = sum(req_pages) + 3
    hkv, d = dims.n_kv_heads, dims.head_dim
    k = synth.to_storage(rng.standard_normal((n_pages, hkv, 16, d)), "bf16")
    v = synth.to_storage(rng.standard_normal((n_pages, hkv, d, 16)), "bf16")
    perm = rng.permutation(n_pages).astype(np.int32)
    bt = np.full((len(lens), max(max(req_pages), 1)), -1, np.int32)
    owned = np.zeros((n_pages, 16), bool)
    o = 0
    for r, n in enumerate(lens):
        bt[r, :req_pages[r]] = perm[o:o + req_pages[r]]
        for j in range(n):
            owned[bt[r, j // 16], j % 16] = True
        o += req_pages[r]
    kt = torch.from_numpy(k).to(torch.bfloat16)
    vt = torch.from_numpy(v).to(torch.bfloat16)
    ki, vi = kt.view(torch.int16), vt.view(torch.int16)
    for p in range(n_pages):
        for s in range(16):
            if not owned[p, s]:
                ki[p, :, s, :] = NAN_BF16
                vi[p, :, :, s] = NAN_BF16
    pool = LY.PagePool(kt.to(DEV), vt.to(DEV))
    q = synth.to_storage(rng.standard_normal((len(lens), dims.n_q_heads, d)) * qscale, "bf16")
    return seq, bt, k, v, pool, q


def _run(dims, lens, seed, qscale=1.0):
    seq, bt, kh, vh, pool, q = _case(dims, lens, seed, qscale)
    n_req = len(lens)
    lay = LY.DeviceLayout(seq, bt, LY.rope_table(dims.theta, dims.head_dim, 16, DEV), DEV)
    cd = LY.make_dims(dims)
    o = torch.full((n_req, dims.n_q_heads * dims.head_dim), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((n_req, dims.n_q_heads), dtype=torch.float32, device=DEV)
    ws = LY.workspace(L.SX_OP_DECODE, cd, int(seq[-1]), 0, n_req, DEV)
    L.sx_decode_attn(cd, lay.struct, torch.from_numpy(q).to(torch.bfloat16).to(DEV), pool.struct(), o,
                     lse, ws)
    torch.cuda.synchronize()
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    for r, T in enumerate(lens):
        if T == 0:
            assert np.all(og[r] == 0) and np.all(np.isneginf(lg[r]))
            continue
        pages = bt[r]
        idx = np.arange(T)
        K = kh[pages[idx // 16], :, idx % 16, :]
        V = vh[pages[idx // 16], :, :, idx % 16]
        ref, lref = oracle.causal_attention(q[r:r + 1], np.array([T - 1]), K, V)
        assert_close_bf16(og[r:r + 1], ref.reshape(1, -1), what=f"decode O request {r} (T={T})")
        assert np.max(np.abs(lg[r] - lref[0])) < 2e-3, f"lse request {r}"
    return og


@pytest.mark.parametrize("shape,lens", [
    ("llama", [1, 15, 16, 17, 31, 32, 33, 700]),
    ("llama", [0, 129, 0]),
    ("qwen", [2000, 77, 48]),
])
def test_decode_parity_ragged(shape, lens):
    say(f"[decode] shape={shape} lens={lens}")
    _run(SHAPES[shape], lens, seed=sum(lens) + 5)


def test_decode_parity_sharp_softmax():
    """Large logits: a few keys carry almost all the mass."""
    say("[decode] sharp softmax")
    _run(SHAPES["llama"], [3000, 513], seed=17, qscale=6.0)


@pytest.mark.parametrize("lens", [[31745], [16000, 16001, 15999, 16384]])
def test_decode_parity_full_size(lens):
    """The rag32k request after its prefill (31,744 tokens + the new one),
    and a 4-request batch of ~16K tokens each: every head of every request."""
    say(f"[decode] full size lens={lens}")
    _run(SHAPES["llama"], lens, seed=23)
