"""Per-kernel GPU parity against the CPU oracle on identical seeded inputs.

Every entry point is called through the C ABI (libsx.so) and compared with
the oracle function that defines the same step.  Tolerances:
  fp32 storage: max |g - r| <= 1e-4 * max |r| per tensor;
  bf16 outputs against the unrounded oracle: |g - r| <= 1e-2 + 2^-8 |r|
  (the store itself adds up to half a bf16 step, 2^-8 |r|, which alone
  exceeds 1e-2 for |r| >= 2.56);
  bf16 stored values against the oracle's rounded values: one bf16 step per
  storage rounding, |g - r| <= 1e-2 + 2^-7 |r|;
  integer/index results and page-table writes: bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle
from segment_level_kv_amd import _lib as L
from segment_level_kv_amd import layer as LY
from segment_level_kv_amd import synth
from tests.gpu_util import (BF16_STEP_REL, assert_close_bf16, assert_close_f32, assert_o_bf16, bf16_ulps,
                            say, selection_contract)

pytestmark = pytest.mark.gpu
DEV = "cuda"

SHAPES = {
    "llama": synth.Dims(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, theta=5e5, dtype="bf16"),
    "qwen": synth.Dims(hidden=3584, n_q_heads=28, n_kv_heads=4, head_dim=128, theta=1e6, dtype="bf16"),
    "tiny": synth.Dims(hidden=256, n_q_heads=4, n_kv_heads=1, head_dim=64, theta=1e4, dtype="f32"),
}


def _store(a, dims):
    return synth.to_storage(a, dims.dtype)


def _pool_from_logical(dims, n_pages, seed):
    """Random page pool (values of the storage type) and its host copy."""
    rng = np.random.default_rng(seed)
    k = _store(rng.standard_normal((n_pages, dims.n_kv_heads, 16, dims.head_dim)), dims)
    v = _store(rng.standard_normal((n_pages, dims.n_kv_heads, dims.head_dim, 16)), dims)
    dt = LY.storage_dtype(dims.dtype)
    pool = LY.PagePool(torch.from_numpy(k).to(dt).to(DEV), torch.from_numpy(v).to(dt).to(DEV))
    return pool, k, v


def _logical(kh, vh, page_ids, slot0, n):
    """Host logical [n, Hkv, d] view of tokens slot0.. of a page list."""
    ks, vs = [], []
    for j in range(n):
        p = page_ids[(slot0 + j) // 16]
        s = (slot0 + j) % 16
        ks.append(kh[p, :, s, :])
        vs.append(vh[p, :, :, s])
    return np.stack(ks), np.stack(vs)


def _pool_host(pool):
    return (pool.k.float().cpu().double().numpy(), pool.v.float().cpu().double().numpy())


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


# ------------------------------------------------------------------ realign --

@pytest.mark.parametrize("shape", ["llama", "tiny"])
def test_realign_parity_and_copy_semantics(shape):
    dims = SHAPES[shape]
    say(f"[realign] shape={shape}")
    rng = np.random.default_rng(11)
    n_pages = 96
    pool, kh, vh = _pool_from_logical(dims, n_pages, 12)
    perm = rng.permutation(n_pages).astype(np.int32)
    # source pages 0..39 of perm, destination block table from 40..87, 88.. untouched
    src_ids = perm[:40]
    bt = perm[40:88].reshape(2, 24)
    segs = [dict(req=0, dst_start=0, len=64, p_src=300, src_slot0=0, src_pages_off=0),
            dict(req=0, dst_start=64, len=37, p_src=5, src_slot0=3, src_pages_off=4),
            dict(req=0, dst_start=107, len=16, p_src=107, src_slot0=0, src_pages_off=8),   # delta 0
            dict(req=1, dst_start=5, len=200, p_src=9000, src_slot0=11, src_pages_off=10),
            dict(req=1, dst_start=230, len=20, p_src=0, src_slot0=0, src_pages_off=30)]
    pos_off = np.array([0, 1234], np.int32)
    jobs = L.sx_plan_realign(segs, src_ids, bt, pos_offset=pos_off)
    rope = LY.rope_table(dims.theta, dims.head_dim, 12000, DEV)
    lay = LY.DeviceLayout(np.array([0, 256, 512], np.int32), bt, rope, DEV, pos_offset=pos_off)
    before_k, before_v = _bits(pool.k), _bits(pool.v)
    jt = torch.from_numpy(jobs).to(DEV)
    L.sx_rope_realign(LY.make_dims(dims), lay.struct, pool.struct(), pool.struct(), jt, len(jobs))
    torch.cuda.synchronize()
    ak, av = _pool_host(pool)
    after_k, after_v = _bits(pool.k), _bits(pool.v)
    written = np.zeros((n_pages, 16), dtype=bool)
    for s in segs:
        kc, vc = _logical(kh, vh, src_ids[s["src_pages_off"]:], s["src_slot0"], s["len"])
        p_dst = s["dst_start"] + pos_off[s["req"]]
        kr, vr = oracle.realign_segment(kc, vc, s["p_src"], p_dst, dims.theta, dims.dtype)
        kg, vg = _logical(ak, av, bt[s["req"]], s["dst_start"], s["len"])
        assert np.array_equal(vg, vr), "V must be copied bit-exactly"
        if p_dst == s["p_src"]:
            assert np.array_equal(kg, kr), "delta 0 must copy K bit-exactly"
        if dims.dtype == "bf16":
            assert bf16_ulps(kg, kr).max() <= 1
            assert_close_bf16(kg, kr, rel=BF16_STEP_REL, what="realigned K")
        else:
            assert_close_f32(kg, kr, what="realigned K")
        for j in range(s["len"]):
            t = s["dst_start"] + j
            written[bt[s["req"], t // 16], t % 16] = True
    # sources and every slot no segment maps to are bit-unchanged
    for p in range(n_pages):
        for sl in range(16):
            if not written[p, sl]:
                assert np.array_equal(after_k[p, :, sl], before_k[p, :, sl])
                assert np.array_equal(after_v[p, :, :, sl], before_v[p, :, :, sl])


# ---------------------------------------------------------------- recompute --

@pytest.mark.parametrize("shape,n_rows", [("llama", 300), ("qwen", 130), ("tiny", 40), ("llama", 1),
                                          ("llama", 16), ("llama", 17), ("qwen", 32), ("llama", 48),
                                          ("qwen", 64), ("llama", 65), ("qwen", 257),
                                          ("llama", 513)])
def test_recompute_parity_and_scatter(shape, n_rows):
    dims = SHAPES[shape]
    say(f"[recompute] shape={shape} rows={n_rows}")
    rng = np.random.default_rng(21)
    seq = np.array([0, 700, 1000], np.int32)
    n_tok = int(seq[-1])
    x = _store(synth._rmsnormed_gaussian(rng, n_tok, dims.hidden, dims.eps), dims)
    case_w = synth._weights(rng, dims)
    w = np.concatenate(case_w, axis=0)
    rows = np.sort(rng.choice(n_tok, size=n_rows, replace=False)).astype(np.int32)
    rng.shuffle(rows)                             # row order need not be sorted
    n_pages = 100
    pool = LY.PagePool.alloc(n_pages, dims, DEV)
    perm = rng.permutation(n_pages).astype(np.int32)
    bt = perm[:2 * 44].reshape(2, 44)
    rope = LY.rope_table(dims.theta, dims.head_dim, 1100, DEV)
    pos_off = np.array([0, 77], np.int32)
    lay = LY.DeviceLayout(seq, bt, rope, DEV, pos_offset=pos_off)
    dt = LY.storage_dtype(dims.dtype)
    xt = torch.from_numpy(x).to(dt).to(DEV)
    wt = torch.from_numpy(w).to(dt).to(DEV)
    rt = torch.from_numpy(rows).to(DEV)
    q = torch.full((n_rows, dims.n_q_heads, dims.head_dim), 7.0, dtype=dt, device=DEV)
    before_k, before_v = _bits(pool.k), _bits(pool.v)
    L.sx_recompute_kv(LY.make_dims(dims), lay.struct, xt, rt, n_rows, wt, pool.struct(), q)
    torch.cuda.synchronize()
    req = (rows >= 700).astype(int)
    idx = rows - seq[req]
    pos = idx + pos_off[req]
    qr, kr, vr = oracle.project_rows(x[rows], case_w[0], case_w[1], case_w[2], pos, dims.theta,
                                     dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.dtype)
    qg = q.float().cpu().double().numpy()
    ak, av = _pool_host(pool)
    kg = np.stack([ak[bt[r, i // 16], :, i % 16, :] for r, i in zip(req, idx)])
    vg = np.stack([av[bt[r, i // 16], :, :, i % 16] for r, i in zip(req, idx)])
    if dims.dtype == "bf16":
        for g_, r_, nm in [(qg, qr, "Q"), (kg, kr, "K"), (vg, vr, "V")]:
            # away from zero the two roundings differ by at most one step; near
            # zero cancellation in the dot product makes steps meaningless
            big = np.abs(r_) >= 1e-2
            assert bf16_ulps(g_[big], r_[big]).max() <= 1, nm
            assert_close_bf16(g_, r_, rel=BF16_STEP_REL, what=nm)
    else:
        assert_close_f32(qg, qr, what="Q")
        assert_close_f32(kg, kr, what="K")
        assert_close_f32(vg, vr, what="V")
    # exactly the listed rows' slots were written
    after_k, after_v = _bits(pool.k), _bits(pool.v)
    hit = np.zeros((n_pages, 16), dtype=bool)
    for r, i in zip(req, idx):
        hit[bt[r, i // 16], i % 16] = True
    for p in range(n_pages):
        for sl in range(16):
            if not hit[p, sl]:
                assert np.array_equal(after_k[p, :, sl], before_k[p, :, sl])
                assert np.array_equal(after_v[p, :, :, sl], before_v[p, :, :, sl])


@pytest.mark.parametrize("n_rows", [5200, 3379])
def test_recompute_multi_head_tiles_every_row(n_rows):
    """Row counts whose launch takes multi-head tiles: 5,200 of 6,000 tokens
    in Llama shapes take 256 x 256 tiles (two heads), with Q (48 heads) and
    K/V only (16 heads); 3,379 rows (the rag32k active-set size) take
    256 x 384 tiles (three heads) with Q, one-head tiles K/V only.  The
    oracle projects every row (the last row tile is partial); every head of
    every row is compared, and exactly the listed rows' slots are written."""
    dims = SHAPES["llama"]
    say(f"[recompute] multi-head tiles: rows={n_rows}")
    rng = np.random.default_rng(23)
    seq = np.array([0, 4000, 6000], np.int32)
    n_tok = int(seq[-1])
    x = _store(synth._rmsnormed_gaussian(rng, n_tok, dims.hidden, dims.eps), dims)
    case_w = synth._weights(rng, dims)
    w = np.concatenate(case_w, axis=0)
    rows = np.sort(rng.choice(n_tok, size=n_rows, replace=False)).astype(np.int32)
    rng.shuffle(rows)
    n_pages = 2 * 250 + 8
    perm = rng.permutation(n_pages).astype(np.int32)
    bt = perm[:2 * 250].reshape(2, 250)
    rope = LY.rope_table(dims.theta, dims.head_dim, 6200, DEV)
    pos_off = np.array([0, 131], np.int32)
    lay = LY.DeviceLayout(seq, bt, rope, DEV, pos_offset=pos_off)
    dt = LY.storage_dtype(dims.dtype)
    xt = torch.from_numpy(x).to(dt).to(DEV)
    wt = torch.from_numpy(w).to(dt).to(DEV)
    rt = torch.from_numpy(rows).to(DEV)
    req = (rows >= 4000).astype(int)
    idx = rows - seq[req]
    sample = np.arange(n_rows)
    s_rows = rows[sample]
    qr, kr, vr = oracle.project_rows(x[s_rows], case_w[0], case_w[1], case_w[2],
                                     idx[sample] + pos_off[req[sample]], dims.theta,
                                     dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.dtype)
    for with_q in (True, False):
        pool = LY.PagePool.alloc(n_pages, dims, DEV)
        q = torch.full((n_rows, dims.n_q_heads, dims.head_dim), 7.0, dtype=dt, device=DEV) if with_q else None
        before_k, before_v = _bits(pool.k), _bits(pool.v)
        L.sx_recompute_kv(LY.make_dims(dims), lay.struct, xt, rt, n_rows, wt, pool.struct(), q)
        torch.cuda.synchronize()
        ak, av = _pool_host(pool)
        kg = np.stack([ak[bt[r, i // 16], :, i % 16, :] for r, i in zip(req[sample], idx[sample])])
        vg = np.stack([av[bt[r, i // 16], :, :, i % 16] for r, i in zip(req[sample], idx[sample])])
        pairs = [(kg, kr, "K"), (vg, vr, "V")]
        if with_q:
            pairs.append((q.float().cpu().double().numpy()[sample], qr, "Q"))
        for g_, r_, nm in pairs:
            big = np.abs(r_) >= 1e-2
            assert bf16_ulps(g_[big], r_[big]).max() <= 1, nm
            assert_close_bf16(g_, r_, rel=BF16_STEP_REL, what=f"{nm} (with_q={with_q})")
        after_k, after_v = _bits(pool.k), _bits(pool.v)
        hit = np.zeros((n_pages, 16), dtype=bool)
        hit[bt[req, idx // 16], idx % 16] = True
        changed_k = np.any(after_k != before_k, axis=(1, 3))          # [page, slot]
        changed_v = np.any(after_v != before_v, axis=(1, 2))
        assert not np.any(changed_k & ~hit) and not np.any(changed_v & ~hit)


@pytest.mark.parametrize("n_rows", [3379, 1500, 40, 6000])
def test_recompute_with_next_realign_equals_two_calls(n_rows):
    """sx_recompute_kv_realign (layer l's projection carrying layer l+1's
    realign) gives the same bits as sx_recompute_kv followed by
    sx_rope_realign: Q, the projection's pool and the realign destination
    pool.  3,379 and 1,500 rows run the realign jobs on the compute units the
    projection's tiles leave free (one launch); 40 rows (the few-rows kernel)
    and 6,000 rows (more than one round of tiles) launch the two kernels one
    after the other.  The jobs include full pages, partial slot ranges and
    negative deltas."""
    dims = SHAPES["llama"]
    say(f"[recompute+realign] rows={n_rows}")
    rng = np.random.default_rng(29)
    seq = np.array([0, 4000, 6000], np.int32)
    n_tok = int(seq[-1])
    dt = LY.storage_dtype(dims.dtype)
    x = torch.from_numpy(_store(synth._rmsnormed_gaussian(rng, n_tok, dims.hidden, dims.eps), dims)).to(dt).to(DEV)
    w = torch.from_numpy(np.concatenate(synth._weights(rng, dims), axis=0)).to(dt).to(DEV)
    rows = torch.from_numpy(np.sort(rng.choice(n_tok, size=n_rows, replace=False)).astype(np.int32)).to(DEV)
    n_pages = 2 * 250 + 8
    bt = rng.permutation(n_pages).astype(np.int32)[:500].reshape(2, 250)
    rope = LY.rope_table(dims.theta, dims.head_dim, 6200, DEV)
    lay = LY.DeviceLayout(seq, bt, rope, DEV)
    cd = LY.make_dims(dims)
    src = LY.PagePool.alloc(n_pages, dims, DEV, fill_guard=False)
    g = torch.Generator(device=DEV)
    g.manual_seed(31)
    src.k.copy_(torch.randn(src.k.shape, generator=g, device=DEV).to(dt))
    src.v.copy_(torch.randn(src.v.shape, generator=g, device=DEV).to(dt))
    jobs_h = []
    for p in range(400):
        d = int(rng.integers(-3000, 3000))
        if p % 7 == 3:
            s0, d0, n = int(rng.integers(0, 8)), int(rng.integers(0, 8)), int(rng.integers(1, 9))
        else:
            s0, d0, n = 0, 0, 16
        jobs_h.append((int(rng.integers(0, n_pages)), int(bt.reshape(-1)[p]), s0, d0, n, d))
    jobs = torch.tensor(jobs_h, dtype=torch.int32, device=DEV)

    def fresh():
        kv = LY.PagePool.alloc(n_pages, dims, DEV)
        dst = LY.PagePool.alloc(n_pages, dims, DEV)
        q = torch.full((n_rows, dims.n_q_heads, dims.head_dim), 7.0, dtype=dt, device=DEV)
        return kv, dst, q

    kv_a, dst_a, q_a = fresh()
    L.sx_recompute_kv(cd, lay.struct, x, rows, n_rows, w, kv_a.struct(), q_a)
    L.sx_rope_realign(cd, lay.struct, src.struct(), dst_a.struct(), jobs, len(jobs_h))
    kv_b, dst_b, q_b = fresh()
    L.sx_recompute_kv_realign(cd, lay.struct, x, rows, n_rows, w, kv_b.struct(), q_b, src.struct(),
                              dst_b.struct(), jobs, len(jobs_h))
    torch.cuda.synchronize()
    for a, b, nm in [(q_a, q_b, "Q"), (kv_a.k, kv_b.k, "K pool"), (kv_a.v, kv_b.v, "V pool"),
                     (dst_a.k, dst_b.k, "realigned K pool"), (dst_a.v, dst_b.v, "realigned V pool")]:
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), nm
    assert not torch.equal(dst_b.k.view(torch.int16), LY.PagePool.alloc(n_pages, dims, DEV).k.view(torch.int16))


# ---------------------------------------------------------------- attention --

def _attn_inputs(dims, lens, seed):
    rng = np.random.default_rng(seed)
    seq = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    req_pages = [(n + 15) // 16 for n in lens]
    n_pages = sum(req_pages) + 4
    pool, kh, vh = _pool_from_logical(dims, n_pages, seed + 1)
    perm = rng.permutation(n_pages).astype(np.int32)
    bt = np.full((len(lens), max(req_pages)), -1, np.int32)
    o = 0
    for r, n in enumerate(req_pages):
        bt[r, :n] = perm[o:o + n]
        o += n
    return rng, seq, pool, kh, vh, bt


@pytest.mark.parametrize("shape,lens,density,qscale", [
    ("llama", [700, 333], 0.3, 1.0),
    ("llama", [1500], 0.12, 3.0),
    ("qwen", [650, 90], 0.4, 2.0),
    ("tiny", [144, 50], 0.5, 1.0),
])
def test_sparse_attention_parity(shape, lens, density, qscale):
    dims = SHAPES[shape]
    say(f"[attn] shape={shape} lens={lens} density={density}")
    rng, seq, pool, kh, vh, bt = _attn_inputs(dims, lens, 31)
    rows, starts = [], [0]
    for r, n in enumerate(lens):
        sel = np.flatnonzero(rng.random(n) < density)
        sel = np.union1d(sel, [0, n - 1])                      # first and last token included
        rows.append(sel + seq[r])
        starts.append(starts[-1] + len(sel))
    rows = np.concatenate(rows).astype(np.int32)
    n_rows = len(rows)
    q = _store(rng.standard_normal((n_rows, dims.n_q_heads, dims.head_dim)) * qscale, dims)
    dt = LY.storage_dtype(dims.dtype)
    rope = LY.rope_table(dims.theta, dims.head_dim, 16, DEV)
    lay = LY.DeviceLayout(seq, bt, rope, DEV)
    cd = LY.make_dims(dims)
    o = torch.zeros((n_rows, dims.n_q_heads * dims.head_dim), dtype=dt, device=DEV)
    lse = torch.zeros((n_rows, dims.n_q_heads), dtype=torch.float32, device=DEV)
    ws = LY.workspace(L.SX_OP_SPARSE_ATTN, cd, int(seq[-1]), n_rows, len(lens), DEV)
    L.sx_sparse_attn(cd, lay.struct, torch.from_numpy(q).to(dt).to(DEV), torch.from_numpy(rows).to(DEV),
                     torch.from_numpy(np.array(starts, np.int32)).to(DEV), n_rows, pool.struct(), o, lse, ws)
    torch.cuda.synchronize()
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    for r in range(len(lens)):
        K, V = _logical(kh, vh, bt[r], 0, lens[r])
        sl = slice(starts[r], starts[r + 1])
        ref, lref = oracle.causal_attention(q[sl], rows[sl] - seq[r], K, V)
        ref = ref.reshape(len(ref), -1)
        if dims.dtype == "bf16":
            assert_close_bf16(og[sl], ref, what=f"O req {r}")
            assert np.max(np.abs(lg[sl] - lref)) < 2e-3
        else:
            assert_close_f32(og[sl], ref, what=f"O req {r}")
            assert np.max(np.abs(lg[sl] - lref)) < 1e-4


@pytest.mark.parametrize("shape,lens,density", [("llama", [700, 333], 0.3), ("llama", [3000, 1200], 0.9),
                                                ("tiny", [144, 50], 0.5)])
def test_sparse_attention_plan_then_runs_equal_one_shot(shape, lens, density):
    """sx_sparse_attn_plan once, then sx_sparse_attn_run for two different
    query sets: bit-identical to sx_sparse_attn on each.  The first case has
    few rows (tiles split into key chunks, merge pass), the second enough
    rows that nothing is split, the third is the fp32 path (no work list)."""
    dims = SHAPES[shape]
    say(f"[attn plan/run] shape={shape} lens={lens} density={density}")
    rng, seq, pool, kh, vh, bt = _attn_inputs(dims, lens, 37)
    rows, starts = [], [0]
    for r, n in enumerate(lens):
        sel = np.union1d(np.flatnonzero(rng.random(n) < density), [0, n - 1])
        rows.append(sel + seq[r])
        starts.append(starts[-1] + len(sel))
    rows = np.concatenate(rows).astype(np.int32)
    n_rows = len(rows)
    dt = LY.storage_dtype(dims.dtype)
    rope = LY.rope_table(dims.theta, dims.head_dim, 16, DEV)
    lay = LY.DeviceLayout(seq, bt, rope, DEV)
    cd = LY.make_dims(dims)
    rd = torch.from_numpy(rows).to(DEV)
    sd = torch.from_numpy(np.array(starts, np.int32)).to(DEV)
    qs = [torch.from_numpy(_store(rng.standard_normal((n_rows, dims.n_q_heads, dims.head_dim)), dims)).to(dt).to(DEV)
          for _ in range(2)]
    ws = LY.workspace(L.SX_OP_SPARSE_ATTN, cd, int(seq[-1]), n_rows, len(lens), DEV)
    ws2 = LY.workspace(L.SX_OP_SPARSE_ATTN, cd, int(seq[-1]), n_rows, len(lens), DEV)
    L.sx_sparse_attn_plan(cd, lay.struct, rd, sd, n_rows, ws2)
    for q in qs:
        o1 = torch.zeros((n_rows, dims.n_q_heads * dims.head_dim), dtype=dt, device=DEV)
        o2 = torch.full_like(o1, 7.0)
        l1 = torch.zeros((n_rows, dims.n_q_heads), dtype=torch.float32, device=DEV)
        l2 = torch.full_like(l1, 7.0)
        L.sx_sparse_attn(cd, lay.struct, q, rd, sd, n_rows, pool.struct(), o1, l1, ws)
        L.sx_sparse_attn_run(cd, lay.struct, q, rd, n_rows, pool.struct(), o2, l2, ws2)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16) if dt != torch.float32 else o1.view(torch.int32),
                           o2.view(torch.int16) if dt != torch.float32 else o2.view(torch.int32))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


@pytest.mark.parametrize("shape,lens", [("llama", [900, 130]), ("tiny", [144])])
def test_full_attention_parity(shape, lens):
    dims = SHAPES[shape]
    say(f"[full attn] shape={shape} lens={lens}")
    rng, seq, pool, kh, vh, bt = _attn_inputs(dims, lens, 41)
    n_tok = int(seq[-1])
    q = _store(rng.standard_normal((n_tok, dims.n_q_heads, dims.head_dim)), dims)
    dt = LY.storage_dtype(dims.dtype)
    lay = LY.DeviceLayout(seq, bt, LY.rope_table(dims.theta, dims.head_dim, 16, DEV), DEV)
    cd = LY.make_dims(dims)
    o = torch.zeros((n_tok, dims.n_q_heads * dims.head_dim), dtype=dt, device=DEV)
    lse = torch.full((n_tok, dims.n_q_heads), 7.0, dtype=torch.float32, device=DEV)
    ws = LY.workspace(L.SX_OP_FULL_ATTN, cd, n_tok, n_tok, len(lens), DEV)
    L.sx_full_attn(cd, lay.struct, torch.from_numpy(q).to(dt).to(DEV), pool.struct(), o, lse, ws)
    torch.cuda.synchronize()
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    for r in range(len(lens)):
        K, V = _logical(kh, vh, bt[r], 0, lens[r])
        sl = slice(seq[r], seq[r + 1])
        ref, lse_ref = oracle.causal_attention(q[sl], np.arange(lens[r]), K, V)
        ref = ref.reshape(len(ref), -1)
        # the normaliser is fp32 on the GPU over the same stored q and K
        lerr = float(np.max(np.abs(lg[sl] - lse_ref)))
        assert lerr <= 1e-4, f"LSE req {r}: max abs err {lerr:.3g}"
        if dims.dtype == "bf16":
            err = assert_o_bf16(og[sl], ref, what=f"O req {r}")
        else:
            err = assert_close_f32(og[sl], ref, what=f"O req {r}")
        say(f"  req {r}: O max err {err:.3g} LSE max abs err {lerr:.3g}")


# ------------------------------------------------------------ probe + top-k --

@pytest.mark.parametrize("shape,lens,n_new", [("llama", [1200, 500], 70), ("qwen", [800], 40),
                                              ("tiny", [144, 60], 16)])
def test_select_topk_parity(shape, lens, n_new):
    dims = SHAPES[shape]
    say(f"[select] shape={shape} lens={lens}")
    rng, seq, pool, kh, vh, bt = _attn_inputs(dims, lens, 51)
    n_tok = int(seq[-1])
    tok_class = np.zeros(n_tok, np.uint8)
    sq_rows, sq_start, ks = [], [0], []
    for r, n in enumerate(lens):
        sq = np.union1d(np.arange(n - n_new, n), rng.choice(n, size=n_new // 4, replace=False))
        tok_class[sq + seq[r]] = 1
        sq_rows.append(sq + seq[r])
        sq_start.append(sq_start[-1] + len(sq))
        ks.append(int(0.2 * (n - len(sq))))
    sq_rows = np.concatenate(sq_rows).astype(np.int32)
    n_sq = len(sq_rows)
    q = _store(rng.standard_normal((n_sq, dims.n_q_heads, dims.head_dim)) * 2.0, dims)
    dt = LY.storage_dtype(dims.dtype)
    lay = LY.DeviceLayout(seq, bt, LY.rope_table(dims.theta, dims.head_dim, 16, DEV), DEV)
    cd = LY.make_dims(dims)
    k_sel = np.array(ks, np.int32)
    sel = torch.full((int(k_sel.sum()),), -7, dtype=torch.int32, device=DEV)
    act = torch.full((n_sq + int(k_sel.sum()),), -7, dtype=torch.int32, device=DEV)
    scores = torch.zeros(n_tok, dtype=torch.float32, device=DEV)
    ws = LY.workspace(L.SX_OP_SELECT, cd, n_tok, n_sq, len(lens), DEV)
    L.sx_select_topk(cd, lay.struct, torch.from_numpy(q).to(dt).to(DEV), None,
                     torch.from_numpy(sq_rows).to(DEV), torch.from_numpy(np.array(sq_start, np.int32)).to(DEV),
                     n_sq, None, pool.struct(), torch.from_numpy(tok_class).to(DEV),
                     torch.from_numpy(k_sel).to(DEV), sel, act, scores, ws)
    torch.cuda.synchronize()
    sg = scores.cpu().double().numpy()
    selg = sel.cpu().numpy()
    actg = act.cpu().numpy()
    off = 0
    for r, n in enumerate(lens):
        K, _ = _logical(kh, vh, bt[r], 0, n)
        sl = slice(sq_start[r], sq_start[r + 1])
        qpos = sq_rows[sl] - seq[r]
        _, lse = oracle.causal_attention(q[sl], qpos, K, K)
        ref = oracle.attention_mass_scores(q[sl], qpos, K, lse)
        got = sg[seq[r]:seq[r + 1]]
        tol = 2e-5 * ref.max()
        err = np.abs(got - ref)
        assert np.all(err <= 1e-4 * ref + tol), f"scores: max rel err {np.max(err / (ref + tol)):.3g}"
        cand = np.flatnonzero(tok_class[seq[r]:seq[r + 1]] == 0)
        gsel = selg[off:off + ks[r]] - seq[r]
        assert np.all(np.diff(gsel) > 0), "selection must be ascending"
        ndiff = selection_contract(gsel, ref, cand, ks[r], tol + 1e-4 * ref.max())
        # active set = Sparse-Q rows merged with the selection, ascending
        a_off = sq_start[r] + off
        ga = actg[a_off:a_off + len(qpos) + ks[r]] - seq[r]
        assert np.array_equal(ga, np.union1d(qpos, gsel))
        say(f"  req {r}: k={ks[r]} differing indices={ndiff}")
        off += ks[r]


def test_topk_bit_exact_adversarial():
    """Top-k on identical scores must equal the oracle bit for bit,
    including all-equal scores, two-valued scores and signed zeros."""
    say("[topk] adversarial")
    rng = np.random.default_rng(61)
    lens = [3000, 1, 700, 5000, 2048, 100]
    seq = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n_tok = int(seq[-1])
    parts = [rng.standard_normal(3000).astype(np.float32), np.zeros(1, np.float32),
             np.full(700, 0.5, np.float32),
             np.where(rng.random(5000) < 0.5, 2.0, 1.0).astype(np.float32),
             np.where(rng.random(2048) < 0.5, 0.0, -0.0).astype(np.float32),
             (np.round(rng.random(100) * 3) / 4).astype(np.float32)]
    scores = np.concatenate(parts)
    tok_class = (rng.random(n_tok) < 0.2).astype(np.uint8)
    ks = [1000, 1, 333, 2500, 900, 0]
    n_cand = [int(np.sum(tok_class[seq[r]:seq[r + 1]] == 0)) for r in range(len(lens))]
    ks = [min(k, c) for k, c in zip(ks, n_cand)]
    sel = torch.full((sum(ks),), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(L.sx_workspace_bytes(L.SX_OP_TOPK, LY.make_dims(SHAPES["llama"]), n_tok, 0, len(lens)),
                     dtype=torch.uint8, device=DEV)
    L.sx_topk(torch.from_numpy(scores).to(DEV), torch.from_numpy(tok_class).to(DEV),
              torch.from_numpy(seq).to(DEV), len(lens), n_tok, torch.from_numpy(np.array(ks, np.int32)).to(DEV),
              sel, ws)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    off = 0
    for r in range(len(lens)):
        sc = scores[seq[r]:seq[r + 1]].astype(np.float64)
        cand = np.flatnonzero(tok_class[seq[r]:seq[r + 1]] == 0)
        ref = oracle.select_topk(sc, cand, ks[r])
        assert np.array_equal(got[off:off + ks[r]] - seq[r], ref), f"request {r}"
        off += ks[r]


def test_topk_many_chunks_ties_and_padding():
    """The radix select runs one workgroup per 1,024-token chunk: ties at
    the threshold that straddle chunk boundaries must still go to the lowest
    token ids, budgets above the candidate count are padded with -1 (also
    for a request with no tokens), and a 70K-token request spans 69 chunks."""
    say("[topk] many chunks, ties, padding")
    rng = np.random.default_rng(67)
    lens = [70000, 0, 1500, 3000, 1025]
    seq = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n_tok = int(seq[-1])
    parts = [rng.integers(0, 6, 70000).astype(np.float32) / 8,      # six values: long tie runs
             np.zeros(0, np.float32),
             rng.standard_normal(1500).astype(np.float32),
             np.where(rng.random(3000) < 0.999, 1.0, 3.0).astype(np.float32),
             np.full(1025, -2.5, np.float32)]
    scores = np.concatenate(parts)
    tok_class = (rng.random(n_tok) < 0.1).astype(np.uint8)
    tok_class[seq[2]:seq[3]] = np.where(rng.random(1500) < 0.9, 2, tok_class[seq[2]:seq[3]])
    n_cand = [int(np.sum(tok_class[seq[r]:seq[r + 1]] == 0)) for r in range(len(lens))]
    k_req = [31000, 5, n_cand[2] + 40, 2999, 1000]
    sel = torch.full((sum(k_req),), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(L.sx_workspace_bytes(L.SX_OP_TOPK, LY.make_dims(SHAPES["llama"]), n_tok, 0, len(lens)),
                     dtype=torch.uint8, device=DEV)
    L.sx_topk(torch.from_numpy(scores).to(DEV), torch.from_numpy(tok_class).to(DEV),
              torch.from_numpy(seq).to(DEV), len(lens), n_tok,
              torch.from_numpy(np.array(k_req, np.int32)).to(DEV), sel, ws)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    off = 0
    for r in range(len(lens)):
        k = min(k_req[r], n_cand[r])
        sc = scores[seq[r]:seq[r + 1]].astype(np.float64)
        cand = np.flatnonzero(tok_class[seq[r]:seq[r + 1]] == 0)
        ref = oracle.select_topk(sc, cand, k)
        seg = got[off:off + k_req[r]]
        assert np.array_equal(seg[:k] - seq[r], ref), f"request {r}"
        assert np.all(seg[k:] == -1), f"request {r}: padding"
        say(f"  req {r}: len {lens[r]} candidates {n_cand[r]} budget {k_req[r]} -> {k} selected")
        off += k_req[r]


def test_select_padding_of_active_rows():
    """sx_select_topk with budgets above the candidate count: the selection
    and the active rows (Sparse-Q rows merged with the selection) are padded
    with -1 after their valid entries."""
    dims = SHAPES["llama"]
    lens = [900, 0, 2100]
    say(f"[select] padding lens={lens}")
    rng, seq, pool, kh, vh, bt = _attn_inputs(dims, lens, 71)
    cd = LY.make_dims(dims)
    n_tok = int(seq[-1])
    lay = LY.DeviceLayout(np.asarray(seq, np.int32), bt, LY.rope_table(dims.theta, dims.head_dim, 4096, DEV), DEV)
    sq_rows = np.r_[seq[0] + 880:seq[0] + 900, seq[2] + 2000:seq[2] + 2100].astype(np.int32)
    sq_start = np.array([0, 20, 20, 120], np.int32)
    tok_class = np.where(rng.random(n_tok) < 0.5, 2, 0).astype(np.uint8)
    tok_class[sq_rows] = 1
    n_cand = [int(np.sum(tok_class[seq[r]:seq[r + 1]] == 0)) for r in range(len(lens))]
    k_req = np.array([n_cand[0] + 7, 3, 50], np.int32)
    q = (rng.standard_normal((len(sq_rows), dims.n_q_heads, dims.head_dim)) * 0.5).astype(np.float32)
    sel = torch.full((int(k_req.sum()),), -7, dtype=torch.int32, device=DEV)
    act = torch.full((len(sq_rows) + int(k_req.sum()),), -7, dtype=torch.int32, device=DEV)
    ws = LY.workspace(L.SX_OP_SELECT, cd, n_tok, len(sq_rows), len(lens), DEV)
    L.sx_select_topk(cd, lay.struct, torch.from_numpy(q).to(torch.bfloat16).to(DEV), None,
                     torch.from_numpy(sq_rows).to(DEV), torch.from_numpy(sq_start).to(DEV), len(sq_rows),
                     None, pool.struct(), torch.from_numpy(tok_class).to(DEV), torch.from_numpy(k_req).to(DEV),
                     sel, act, None, ws)
    torch.cuda.synchronize()
    selg, actg = sel.cpu().numpy(), act.cpu().numpy()
    off = 0
    for r in range(len(lens)):
        k = min(int(k_req[r]), n_cand[r])
        s = selg[off:off + k_req[r]]
        assert np.all(np.diff(s[:k]) > 0) and np.all(s[k:] == -1), f"request {r}: selection {s}"
        n_sq = sq_start[r + 1] - sq_start[r]
        a = actg[sq_start[r] + off:sq_start[r] + off + n_sq + k_req[r]]
        assert np.array_equal(a[:n_sq + k], np.union1d(sq_rows[sq_start[r]:sq_start[r + 1]], s[:k])), r
        assert np.all(a[n_sq + k:] == -1), f"request {r}: active rows {a}"
        off += k_req[r]
    assert np.all(selg != -7) and np.all(actg != -7)


def test_sparse_attention_rows_far_apart():
    """A handful of active rows at the start and at the end of a long
    request share query tiles: the tiles are split on the key grid, and for
    the early rows most chunks lie wholly past their position (empty
    partials that the merge must weigh with 0).  The LSE-only probe pass is
    checked on the same rows."""
    dims = SHAPES["llama"]
    lens = [20000, 700]
    say(f"[attn far apart] lens={lens}")
    rng, seq, pool, kh, vh, bt = _attn_inputs(dims, lens, 91)
    sel0 = np.r_[0:40, 19960:20000]
    sel1 = np.r_[3:9, 690:700]
    rows = np.concatenate([sel0 + seq[0], sel1 + seq[1]]).astype(np.int32)
    starts = [0, len(sel0), len(sel0) + len(sel1)]
    n_rows = len(rows)
    q = _store(rng.standard_normal((n_rows, dims.n_q_heads, dims.head_dim)) * 2.0, dims)
    dt = LY.storage_dtype(dims.dtype)
    lay = LY.DeviceLayout(seq, bt, LY.rope_table(dims.theta, dims.head_dim, 16, DEV), DEV)
    cd = LY.make_dims(dims)
    qd = torch.from_numpy(q).to(dt).to(DEV)
    rd = torch.from_numpy(rows).to(DEV)
    sd = torch.from_numpy(np.array(starts, np.int32)).to(DEV)
    o = torch.zeros((n_rows, dims.n_q_heads * dims.head_dim), dtype=dt, device=DEV)
    lse = torch.zeros((n_rows, dims.n_q_heads), dtype=torch.float32, device=DEV)
    ws = LY.workspace(L.SX_OP_SPARSE_ATTN, cd, int(seq[-1]), n_rows, len(lens), DEV)
    L.sx_sparse_attn(cd, lay.struct, qd, rd, sd, n_rows, pool.struct(), o, lse, ws)
    # the selection's internal probe: LSE only (Sparse-Q rows = these rows)
    n_tok = int(seq[-1])
    tok_class = torch.zeros(n_tok, dtype=torch.uint8, device=DEV)
    tok_class[rd.long()] = 1
    k_sel = torch.zeros(len(lens), dtype=torch.int32, device=DEV)
    sel_rows = torch.empty(1, dtype=torch.int32, device=DEV)
    scores = torch.empty(n_tok, dtype=torch.float32, device=DEV)
    ws2 = LY.workspace(L.SX_OP_SELECT, cd, n_tok, n_rows, len(lens), DEV)
    L.sx_select_topk(cd, lay.struct, qd, None, rd, sd, n_rows, None, pool.struct(), tok_class, k_sel,
                     sel_rows, None, scores, ws2)
    torch.cuda.synchronize()
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    sg = scores.cpu().double().numpy()
    for r in range(len(lens)):
        K, V = _logical(kh, vh, bt[r], 0, lens[r])
        sl = slice(starts[r], starts[r + 1])
        pos = rows[sl] - seq[r]
        ref, lref = oracle.causal_attention(q[sl], pos, K, V)
        assert_close_bf16(og[sl], ref.reshape(len(ref), -1), what=f"O req {r}")
        assert np.max(np.abs(lg[sl] - lref)) < 2e-3
        # mass scores over this request's tokens: each row and head gives mass 1 in total
        s_ref = oracle.attention_mass_scores(q[sl], pos, K, lref)
        s_got = sg[seq[r]:seq[r + 1]]
        assert np.all(np.abs(s_got - s_ref) <= 2e-3 * s_ref + 1e-4 * s_ref.max())
        assert abs(s_got.sum() - len(pos) * dims.n_q_heads) < 1e-2 * len(pos) * dims.n_q_heads


@pytest.mark.parametrize("shape", ["llama", "qwen"])
def test_sparse_attention_many_chunks_and_nan_tail(shape):
    """Long requests with few active rows: every query tile is split into
    many key chunks (merged afterwards); the slots past each request's last
    token hold NaN, which must never reach the output."""
    dims = SHAPES[shape]
    lens = [9000, 2100]
    say(f"[attn chunks] shape={shape} lens={lens}")
    rng, seq, pool, kh, vh, bt = _attn_inputs(dims, lens, 71)
    # poison the unused slots of each request's last page (K and V)
    for r, n in enumerate(lens):
        if n % 16:
            pg = int(bt[r, n // 16])
            pool.k[pg, :, n % 16:, :] = float("nan")
            pool.v[pg, :, :, n % 16:] = float("nan")
    rows, starts = [], [0]
    for r, n in enumerate(lens):
        sel = np.flatnonzero(rng.random(n) < 0.03)
        sel = np.union1d(sel, [0, n - 1])
        rows.append(sel + seq[r])
        starts.append(starts[-1] + len(sel))
    rows = np.concatenate(rows).astype(np.int32)
    n_rows = len(rows)
    q = _store(rng.standard_normal((n_rows, dims.n_q_heads, dims.head_dim)) * 1.5, dims)
    dt = LY.storage_dtype(dims.dtype)
    lay = LY.DeviceLayout(seq, bt, LY.rope_table(dims.theta, dims.head_dim, 16, DEV), DEV)
    cd = LY.make_dims(dims)
    o = torch.zeros((n_rows, dims.n_q_heads * dims.head_dim), dtype=dt, device=DEV)
    lse = torch.zeros((n_rows, dims.n_q_heads), dtype=torch.float32, device=DEV)
    ws = LY.workspace(L.SX_OP_SPARSE_ATTN, cd, int(seq[-1]), n_rows, len(lens), DEV)
    L.sx_sparse_attn(cd, lay.struct, torch.from_numpy(q).to(dt).to(DEV), torch.from_numpy(rows).to(DEV),
                     torch.from_numpy(np.array(starts, np.int32)).to(DEV), n_rows, pool.struct(), o, lse, ws)
    torch.cuda.synchronize()
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    for r in range(len(lens)):
        K, V = _logical(kh, vh, bt[r], 0, lens[r])
        sl = slice(starts[r], starts[r + 1])
        ref, lref = oracle.causal_attention(q[sl], rows[sl] - seq[r], K, V)
        assert_close_bf16(og[sl], ref.reshape(len(ref), -1), what=f"O req {r}")
        assert np.max(np.abs(lg[sl] - lref)) < 2e-3


def test_sparse_attention_split_tiles_large_values():
    """Values far beyond fp16's range through split tiles.  Few active rows
    (about 350 of a 3,600-token request) make every tile split into key
    chunks, whose partial outputs are merged; V is the usual random data
    times 2^17 (exact in bf16), so |V| reaches ~5e5.  O scales exactly with
    V, so the bound is the usual one times 2^17."""
    dims = SHAPES["llama"]
    lens = [3600]
    scale = float(2 ** 17)
    say("[attn] split tiles, |V| ~ 1e5")
    rng, seq, pool, kh, vh, bt = _attn_inputs(dims, lens, 57)
    pool.v.mul_(scale)
    vh = vh * scale
    rows = np.union1d(np.flatnonzero(rng.random(lens[0]) < 0.1), [0, lens[0] - 1]).astype(np.int32)
    n_rows = len(rows)
    q = _store(rng.standard_normal((n_rows, dims.n_q_heads, dims.head_dim)), dims)
    rope = LY.rope_table(dims.theta, dims.head_dim, 16, DEV)
    lay = LY.DeviceLayout(seq, bt, rope, DEV)
    cd = LY.make_dims(dims)
    o = torch.zeros((n_rows, dims.n_q_heads * dims.head_dim), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((n_rows, dims.n_q_heads), dtype=torch.float32, device=DEV)
    ws = LY.workspace(L.SX_OP_SPARSE_ATTN, cd, int(seq[-1]), n_rows, 1, DEV)
    L.sx_sparse_attn(cd, lay.struct, torch.from_numpy(q).to(torch.bfloat16).to(DEV),
                     torch.from_numpy(rows).to(DEV), torch.tensor([0, n_rows], dtype=torch.int32, device=DEV),
                     n_rows, pool.struct(), o, lse, ws)
    torch.cuda.synchronize()
    og = o.float().cpu().double().numpy()
    K, V = _logical(kh, vh, bt[0], 0, lens[0])
    ref, lref = oracle.causal_attention(q, rows, K, V)
    ref = ref.reshape(n_rows, -1)
    assert np.abs(ref).max() > 65504.0
    assert_close_bf16(og, ref, atol=1e-2 * scale, what="O, |V| ~ 1e5, split tiles")
    assert np.max(np.abs(lse.cpu().double().numpy() - lref)) < 2e-3
