"""The C-ABI library on the CPU: it loads, exports every function include/sx.h
declares, rejects bad arguments before launching anything, and its host
planners agree with the oracle (no GPU needed for any of this)."""

import ctypes as C
import math
import os
import re

import numpy as np
import pytest

import oracle
from segment_level_kv_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "sx.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sx_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = L.lib()
    declared = _header_functions()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(lib, name), f"libsx.so does not export {name}"
    assert sorted(L.EXPORTED) == declared


def _dims(dtype=L.SX_BF16, head_dim=128, hq=32, hkv=8, hidden=4096, page=16):
    return L.Dims(hidden, hq, hkv, head_dim, page, dtype)


FAKE = C.c_void_p(0x1000)      # never dereferenced: validation fails first


def _layout():
    return L.Layout(1, 16, 1, 16, 0x1000, 0x1000, None, 0x1000)


def test_validation_errors_launch_nothing():
    lib = L.lib()
    lay = _layout()
    pages = L.Pages(0x1000, 0x1000, 4)
    # NULL dims
    assert lib.sx_recompute_kv(None, C.byref(lay), FAKE, FAKE, 1, FAKE, C.byref(pages), None, None) == L.SX_EINVAL
    assert "dims" in L.last_error()
    # bf16 with head_dim 64 is not built
    d = _dims(head_dim=64)
    assert lib.sx_sparse_attn(C.byref(d), C.byref(lay), FAKE, FAKE, FAKE, 1, C.byref(pages), FAKE, None,
                              FAKE, 1 << 20, None) == L.SX_EUNSUPPORTED
    assert "head_dim" in L.last_error()
    # page size other than 16
    d = _dims(page=32)
    assert lib.sx_full_attn(C.byref(d), C.byref(lay), FAKE, C.byref(pages), FAKE, None, FAKE, 1 << 20,
                            None) == L.SX_EUNSUPPORTED
    # heads not a multiple
    d = _dims(hq=30)
    assert lib.sx_rope_realign(C.byref(d), C.byref(lay), C.byref(pages), C.byref(pages), FAKE, 1,
                               None) == L.SX_EINVAL
    # workspace too small
    d = _dims()
    assert lib.sx_sparse_attn(C.byref(d), C.byref(lay), FAKE, FAKE, FAKE, 100, C.byref(pages), FAKE,
                              None, FAKE, 8, None) == L.SX_EWORKSPACE
    assert "workspace" in L.last_error()
    assert lib.sx_select_topk(C.byref(d), C.byref(lay), FAKE, None, FAKE, FAKE, 4, None, C.byref(pages),
                              FAKE, FAKE, FAKE, None, None, None, 0, None) == L.SX_EWORKSPACE
    # NULL pool
    bad = L.Pages(0, 0x1000, 4)
    assert lib.sx_recompute_kv(C.byref(d), C.byref(lay), FAKE, FAKE, 1, FAKE, C.byref(bad), None,
                               None) == L.SX_EINVAL
    # negative sizes
    assert lib.sx_recompute_kv(C.byref(d), C.byref(lay), FAKE, FAKE, -1, FAKE, C.byref(pages), None,
                               None) == L.SX_EINVAL
    bad_lay = L.Layout(0, 16, 1, 16, 0x1000, 0x1000, None, 0x1000)
    assert lib.sx_recompute_kv(C.byref(d), C.byref(bad_lay), FAKE, FAKE, 1, FAKE, C.byref(pages), None,
                               None) == L.SX_EINVAL
    assert lib.sx_topk(None, FAKE, FAKE, 1, 4, FAKE, FAKE, None, 0, None) == L.SX_EINVAL
    # projection + next layer's realign: the realign destination must be another pool
    other = L.Pages(0x2000, 0x3000, 4)
    assert lib.sx_recompute_kv_realign(C.byref(d), C.byref(lay), FAKE, FAKE, 1, FAKE, C.byref(pages), None,
                                       C.byref(other), C.byref(pages), FAKE, 1, None) == L.SX_EINVAL
    assert "another pool" in L.last_error()
    assert lib.sx_recompute_kv_realign(C.byref(d), C.byref(lay), FAKE, FAKE, 1, FAKE, C.byref(pages), None,
                                       C.byref(other), C.byref(other), None, 1, None) == L.SX_EINVAL
    assert lib.sx_recompute_kv_realign(C.byref(d), C.byref(lay), FAKE, FAKE, 1, FAKE, C.byref(pages), None,
                                       C.byref(pages), C.byref(bad), FAKE, 1, None) == L.SX_EINVAL
    # plan / run halves of the sparse attention
    assert lib.sx_sparse_attn_plan(C.byref(d), C.byref(lay), None, FAKE, 4, FAKE, 1 << 20, None) == L.SX_EINVAL
    assert lib.sx_sparse_attn_plan(C.byref(d), C.byref(lay), FAKE, FAKE, 100, FAKE, 8, None) == L.SX_EWORKSPACE
    assert lib.sx_sparse_attn_run(C.byref(d), C.byref(lay), FAKE, FAKE, 100, C.byref(pages), FAKE, None,
                                  FAKE, 8, None) == L.SX_EWORKSPACE
    assert lib.sx_sparse_attn_run(C.byref(d), C.byref(lay), None, FAKE, 4, C.byref(pages), FAKE, None,
                                  FAKE, 1 << 20, None) == L.SX_EINVAL
    assert lib.sx_sparse_attn_run(C.byref(d), C.byref(lay), FAKE, FAKE, -1, C.byref(pages), FAKE, None,
                                  FAKE, 1 << 20, None) == L.SX_EINVAL
    # MFMA probe: sizes and output are checked before any launch
    assert lib.sx_mfma_peak_probe(0, 10, 0, FAKE, None) == L.SX_EINVAL
    assert lib.sx_mfma_peak_probe(4, 0, 1, FAKE, None) == L.SX_EINVAL
    assert lib.sx_mfma_peak_probe(4, 10, 0, None, None) == L.SX_EINVAL
    assert "sx_mfma_peak_probe" in L.last_error()
    # a layout with tokens but no block-table columns
    empty_bt = L.Layout(1, 16, 0, 16, 0x1000, 0x1000, None, 0x1000)
    assert lib.sx_full_attn(C.byref(d), C.byref(empty_bt), FAKE, C.byref(pages), FAKE, None, FAKE,
                            1 << 20, None) == L.SX_EINVAL
    assert "max_pages" in L.last_error()
    assert lib.sx_decode_attn_noalloc(C.byref(d), C.byref(empty_bt), FAKE, C.byref(pages), FAKE, None,
                                      None) == L.SX_EINVAL


def test_zero_sized_calls_are_noops():
    lib = L.lib()
    d = _dims()
    lay = _layout()
    pages = L.Pages(0x1000, 0x1000, 4)
    assert lib.sx_recompute_kv(C.byref(d), C.byref(lay), None, None, 0, None, C.byref(pages), None, None) == 0
    assert lib.sx_sparse_attn(C.byref(d), C.byref(lay), None, None, None, 0, C.byref(pages), None, None,
                              None, 0, None) == 0
    assert lib.sx_rope_realign(C.byref(d), C.byref(lay), C.byref(pages), C.byref(pages), None, 0, None) == 0
    other = L.Pages(0x2000, 0x3000, 4)
    assert lib.sx_recompute_kv_realign(C.byref(d), C.byref(lay), None, None, 0, None, C.byref(pages), None,
                                       C.byref(pages), C.byref(other), None, 0, None) == 0
    assert lib.sx_sparse_attn_plan(C.byref(d), C.byref(lay), None, None, 0, None, 0, None) == 0
    assert lib.sx_sparse_attn_run(C.byref(d), C.byref(lay), None, None, 0, C.byref(pages), None, None,
                                  None, 0, None) == 0


def test_workspace_sizes_are_monotone():
    d = _dims()
    a = L.sx_workspace_bytes(L.SX_OP_SELECT, d, 4352, 256, 1)
    b = L.sx_workspace_bytes(L.SX_OP_SELECT, d, 31488, 256, 1)
    assert 0 < a < b
    assert L.sx_workspace_bytes(L.SX_OP_SPARSE_ATTN, d, 31488, 3379, 1) > 0
    assert L.sx_workspace_bytes(L.SX_OP_RECOMPUTE, d, 31488, 3379, 1) == 0


# ----------------------------------------------------------- host planners --

def test_rope_table_matches_float64_angles():
    tab = L.sx_rope_table(5e5, 128, 2000).astype(np.float64)
    m = np.arange(2000)[:, None]
    om = oracle.rope_inv_freq(128, 5e5)[None, :]
    assert np.max(np.abs(tab[..., 0] - np.cos(m * om))) < 1e-7
    assert np.max(np.abs(tab[..., 1] - np.sin(m * om))) < 1e-7
    big = L.sx_rope_table(1e6, 128, 131200).astype(np.float64)
    mm = 131199
    ref = np.cos(mm * oracle.rope_inv_freq(128, 1e6))
    assert np.max(np.abs(big[mm, :, 0] - ref)) < 1e-7   # fp64-formed angles: no fp32 angle error
    with pytest.raises(L.SxError):
        L.sx_rope_table(-1.0, 128, 10)


@pytest.mark.parametrize("overflow", [0, 16, 5])
def test_plan_layout_matches_oracle_random_batches(overflow):
    rng = np.random.default_rng(5 + overflow)
    for _ in range(100):
        n_req = int(rng.integers(1, 5))
        reqs, pieces_list, ratios = [], [], []
        for _ in range(n_req):
            pieces = [(("reuse", "new")[rng.integers(2)], int(rng.integers(0, 150)))
                      for _ in range(rng.integers(1, 6))]
            ratio = (int(rng.integers(0, 1001)), 1000)
            pieces_list.append(pieces)
            ratios.append(ratio)
            reqs.append(([(k == "reuse", n) for k, n in pieces], ratio))
        got = L.sx_plan_layout(reqs, overflow_tokens=overflow)
        off = 0
        for r in range(n_req):
            ref = oracle.plan_request(pieces_list[r], ratios[r], overflow_tokens=overflow)
            T = ref["T"]
            assert got["seq_start"][r + 1] - got["seq_start"][r] == T
            cls = got["tok_class"][off:off + T]
            assert np.array_equal(np.flatnonzero(cls == 1), ref["sq"])
            assert np.array_equal(np.flatnonzero(cls == 0), ref["cand"])
            sq = got["sq_rows"][got["sq_start"][r]:got["sq_start"][r + 1]] - off
            assert np.array_equal(sq, ref["sq"])
            assert got["k"][r] == ref["k"] and got["n_cand"][r] == len(ref["cand"])
            off += T


def test_decode_validation():
    lib = L.lib()
    lay = _layout()
    pages = L.Pages(0x1000, 0x1000, 4)
    d32 = _dims(dtype=L.SX_F32)
    assert lib.sx_decode_attn(C.byref(d32), C.byref(lay), FAKE, C.byref(pages), FAKE, None, FAKE, 1 << 20,
                              None) == L.SX_EUNSUPPORTED
    d = _dims()
    need = lib.sx_workspace_bytes(L.SX_OP_DECODE, C.byref(d), 16, 0, 1)
    assert need > 0
    assert lib.sx_decode_attn(C.byref(d), C.byref(lay), FAKE, C.byref(pages), FAKE, None, FAKE, need - 1,
                              None) == L.SX_EWORKSPACE
    assert lib.sx_decode_attn(C.byref(d), C.byref(lay), None, C.byref(pages), FAKE, None, FAKE, need,
                              None) == L.SX_EINVAL


def test_plan_layout_rejects_bad_ratio():
    with pytest.raises(L.SxError):
        L.sx_plan_layout([([(True, 10)], (3, 2))])
    with pytest.raises(L.SxError):
        L.sx_plan_layout([([(True, 10)], (1, 0))])
    with pytest.raises(L.SxError):
        L.sx_plan_layout([([(True, 10)], (1, 2))], overflow_tokens=-1)


def test_plan_realign_covers_every_token_once():
    rng = np.random.default_rng(8)
    for _ in range(50):
        n_req = 2
        segs, src_ids = [], []
        bt = rng.permutation(400).astype(np.int32)[:2 * 40].reshape(2, 40)
        src_pool = 1000 + rng.permutation(500).astype(np.int32)
        expected = {}
        for r in range(n_req):
            pos = 0
            for _ in range(rng.integers(1, 5)):
                Ln = int(rng.integers(1, 100))
                s0 = int(rng.integers(0, 16))
                p_src = int(rng.integers(0, 5000))
                off = len(src_ids)
                npg = (s0 + Ln + 15) // 16
                src_ids.extend(src_pool[off:off + npg].tolist())
                segs.append(dict(req=r, dst_start=pos, len=Ln, p_src=p_src, src_slot0=s0, src_pages_off=off))
                for j in range(Ln):
                    expected[(bt[r, (pos + j) // 16], (pos + j) % 16)] = (
                        src_ids[off + (s0 + j) // 16], (s0 + j) % 16, pos - p_src)
                pos += Ln + int(rng.integers(0, 20))
            assert pos <= 40 * 16
        jobs = L.sx_plan_realign(segs, np.array(src_ids, np.int32), bt)
        seen = {}
        for sp, dp, ss, ds, n, delta in jobs:
            assert 1 <= n <= 16 and ss + n <= 16 and ds + n <= 16
            for j in range(n):
                key = (dp, ds + j)
                assert key not in seen
                seen[key] = (sp, ss + j, delta)
        assert seen == expected


def test_plan_realign_rejects_runs_past_the_page_arrays():
    bt = np.arange(4, dtype=np.int32).reshape(1, 4)
    with pytest.raises(L.SxError):
        L.sx_plan_realign([dict(req=0, dst_start=0, len=40, p_src=0, src_pages_off=0)],
                          np.arange(2, dtype=np.int32), bt)
    with pytest.raises(L.SxError):
        L.sx_plan_realign([dict(req=0, dst_start=60, len=10, p_src=0, src_pages_off=0)],
                          np.arange(8, dtype=np.int32), bt)
    with pytest.raises(L.SxError):
        L.sx_plan_realign([dict(req=1, dst_start=0, len=10, p_src=0, src_pages_off=0)],
                          np.arange(8, dtype=np.int32), bt)
