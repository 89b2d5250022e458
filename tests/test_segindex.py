"""Segment lookup in libsx (host C++) against the oracle (CPU only).

The index is host code, so these tests need no GPU: the library's hash is
compared with the published SHA-256 example and with the oracle over every
message length that matters for padding; the index and the segment planner
are driven through random operation sequences on both sides and every
result, error and pool statistic must agree exactly.
"""

import random

import numpy as np
import pytest

from oracle import segindex as si
from segment_level_kv_amd import _lib as L

FIPS_MSG = b"abcdbcdecdefdefgefghfghighijhijkijkljklmklmnlmnomnopnopq"


def test_virtual_hash_fips_example_and_lengths():
    key = int.from_bytes(FIPS_MSG[:8], "little")
    toks = [int.from_bytes(FIPS_MSG[8 + 4 * i:12 + 4 * i], "little", signed=True) for i in range(12)]
    assert L.sx_virtual_hash(toks, key) == int.from_bytes(bytes.fromhex("248d6a61d20638b8"), "little")
    rng = np.random.default_rng(0)
    # message lengths 8 .. 8 + 4*40 bytes: one and two 64-byte blocks, the
    # 55/56/64-byte padding boundaries, negative ids, keys with the top bit set
    for n in range(41):
        t = rng.integers(-2**31, 2**31, n)
        k = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        assert L.sx_virtual_hash(t, k) == si.virtual_hash(t, k), n


def _run_both(seed, n_blocks, bs, num, den, n_ops, vocab):
    rng = random.Random(seed)
    ref = si.BlockIndex(n_blocks, bs, num, den)
    got = L.SegmentIndex(n_blocks, bs, num, den)
    held, cached = [], []

    def both(fn_ref, fn_got):
        try:
            r = fn_ref()
        except (ValueError, MemoryError) as e:
            with pytest.raises(L.SxError) as ei:
                fn_got()
            assert ei.value.status == (L.SX_ENOMEM if isinstance(e, MemoryError) else L.SX_EINVAL)
            return None
        g = fn_got()
        assert g == r
        return r

    for _ in range(n_ops):
        op = rng.random()
        if op < 0.3:
            n = rng.randint(0, 8)
            ids = both(lambda: ref.alloc(n), lambda: got.alloc(n))
            if ids is not None and ids:
                toks = [rng.randint(0, vocab) for _ in range(len(ids) * bs - rng.randint(0, bs - 1))]
                key = rng.randint(0, 3) * (2**62)
                p = rng.randint(0, 1000)
                fr = rng.random() < 0.7
                both(lambda: ref.insert(toks, key, ids, p, fr), lambda: got.insert(toks, key, ids, p, fr))
                cached.append((toks, key))
                held.extend(ids)
        elif op < 0.5 and held:
            k = rng.randint(1, min(3, len(held)))
            pick = [held.pop(rng.randrange(len(held))) for _ in range(k)]
            both(lambda: ref.release(pick), lambda: got.release(pick))
        elif op < 0.8 and cached:
            toks, key = rng.choice(cached)
            if rng.random() < 0.3:   # the segment inside a longer prompt piece, shifted by blocks
                toks = [rng.randint(0, vocab) for _ in range(bs * rng.randint(0, 2))] + toks
            r = both(lambda: ref.lookup(toks, key), lambda: got.lookup(toks, key))
            held.extend(b for b in r[0] if b >= 0)
            # the planner on this lookup
            n_tok = len(toks)
            dst = rng.randint(0, 5) * bs
            off = rng.randint(0, 9)
            segs, ids, pieces = L.sx_plan_segments(2, dst, r[0], r[1], n_tok, bs, off)
            rs, ri, rp = si.plan_segments(2, dst, r[0], r[1], bs, n_tok, off)
            assert segs == rs and ids == ri
            assert pieces == [(k == "reuse", n) for k, n in rp]
        elif op < 0.9:
            # errors: release something not held, remove a free block
            b = rng.randrange(n_blocks)
            both(lambda: ref.release([b] * (ref.ref[b] + 1)),
                 lambda: got.release([b] * (ref.ref[b] + 1)))
        elif held:
            b = rng.choice(held)
            both(lambda: ref.remove([b, b]), lambda: got.remove([b, b]))
        assert got.stats() == ref.stats()
    got.close()


@pytest.mark.parametrize("seed", range(6))
def test_index_matches_oracle_random_sequences(seed):
    """Small pools and a tiny vocabulary: many duplicate blocks, frequent
    eviction and pool exhaustion."""
    _run_both(seed, n_blocks=32, bs=4, num=rng_num(seed), den=10, n_ops=400, vocab=3)


def rng_num(seed):
    return [9, 10, 5, 7, 0, 9][seed]


def test_index_matches_oracle_page_sized_blocks():
    _run_both(99, n_blocks=64, bs=16, num=9, den=10, n_ops=300, vocab=50)


def test_rag_request_end_to_end_lookup():
    """A knowledge base of 17 frozen segments (system prompt + 16 passages,
    padded to whole 16-token blocks) cached at their own offsets; a request
    reorders them and inserts a query: every passage block hits, each
    passage becomes one realign segment with the right delta, and the
    planner's pieces give the layout of the prompt."""
    bs = 16
    rng = np.random.default_rng(3)
    ix = L.SegmentIndex(4096, bs)
    key = 0x5A17
    lens = [512] + [1920] * 16
    segs_tok, segs_ids, segs_pos = [], [], []
    for i, n in enumerate(lens):
        t = rng.integers(0, 128000, n)
        ids = ix.alloc(n // bs)
        p = 0 if i == 0 else 512
        ix.insert(t, key, ids, p, frozen=True)
        ix.release(ids)
        segs_tok.append(t)
        segs_ids.append(ids)
        segs_pos.append(p)
    assert ix.stats() == (sum(lens) // bs, 4096 - sum(lens) // bs, sum(lens) // bs, sum(lens) // bs)
    order = [0] + list(rng.permutation(np.arange(1, 17)))
    dst, off, all_ids, pieces = 0, 0, [], []
    for s in order:
        blk, pos = ix.lookup(segs_tok[s], key)
        assert blk == segs_ids[s] and pos == [segs_pos[s] + j * bs for j in range(len(blk))]
        segs, ids, pc = L.sx_plan_segments(0, dst, blk, pos, lens[s], bs, off)
        assert len(segs) == 1 and segs[0]["len"] == lens[s] and segs[0]["p_src"] == segs_pos[s]
        assert segs[0]["dst_start"] == dst and pc == [(True, lens[s])]
        dst += lens[s]
        off += len(ids)
        all_ids += ids
        pieces += pc
    # the request's query is new: 256 tokens that hit nothing
    q = rng.integers(0, 128000, 256)
    blk, _ = ix.lookup(q, key)
    assert blk == [-1] * 16
    # the hits hold their blocks until released
    assert ix.stats()[0] == sum(lens) // bs
    ix.release(all_ids)
    ix.close()


def test_index_argument_errors():
    with pytest.raises(L.SxError):
        L.SegmentIndex(0, 16)
    with pytest.raises(L.SxError):
        L.SegmentIndex(8, 16, evict_num=11, evict_den=10)
    ix = L.SegmentIndex(8, 4)
    with pytest.raises(L.SxError):
        ix.insert([1, 2, 3, 4], 0, [0], 0, True)      # block 0 not in use
    with pytest.raises(L.SxError) as e:
        ix.alloc(9)
    assert e.value.status == L.SX_ENOMEM
    assert ix.stats() == (0, 8, 0, 0)
    ix.close()
