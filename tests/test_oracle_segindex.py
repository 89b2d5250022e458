"""Pins of the segment-lookup oracle (CPU only).

The hash is pinned to a published SHA-256 example message; the pool and
index semantics to hand-worked scenarios whose expected states are written
out here, and to invariants checked over random operation sequences.
"""

import random

import numpy as np
import pytest

from oracle import segindex as si

# FIPS 180-2 example: the 56-byte message "abcdbcde...nopq" hashes to
# 248d6a61 d20638b8 e5c02693 0c3e6039 a33ce459 64ff2167 f6ecedd4 19db06c1.
FIPS_MSG = b"abcdbcdecdefdefgefghfghighijhijkijkljklmklmnlmnomnopnopq"
FIPS_DIGEST_HEAD = bytes.fromhex("248d6a61d20638b8")


def test_virtual_hash_encoding_on_the_fips_example():
    """Key = first 8 message bytes (little endian), 12 token ids = the other
    48 bytes as little-endian int32: the hash is the digest's first 8 bytes,
    little endian.  A wrong byte order or field width changes the message."""
    key = int.from_bytes(FIPS_MSG[:8], "little")
    toks = [int.from_bytes(FIPS_MSG[8 + 4 * i:12 + 4 * i], "little", signed=True) for i in range(12)]
    assert si.virtual_hash(toks, key) == int.from_bytes(FIPS_DIGEST_HEAD, "little")
    # namespaces (§4.3): same tokens, another key -> another hash
    assert si.virtual_hash(toks, key + 1) != si.virtual_hash(toks, key)


def _toks(n, seed):
    return list(np.random.default_rng(seed).integers(0, 128000, n))


def test_insert_lookup_release_frozen_lifecycle():
    ix = si.BlockIndex(10, 4)
    ids = ix.alloc(3)
    assert ids == [0, 1, 2]
    t = _toks(12, 1)
    ix.insert(t, 7, ids, 100, frozen=True)
    assert ix.stats() == (3, 7, 3, 3)
    ix.release(ids)                               # frozen: stays resident
    assert ix.stats() == (3, 7, 3, 3) and ix.ref[:3] == [0, 0, 0]
    b, p = ix.lookup(t, 7)
    assert b == [0, 1, 2] and p == [100, 104, 108]
    assert ix.ref[:3] == [1, 1, 1] and ix.hits[:3] == [1, 1, 1]
    assert ix.lookup(t, 8) == ([-1] * 3, [-1] * 3)          # other namespace
    assert ix.lookup(t[2:] + t[:2], 7) == ([-1] * 3, [-1] * 3)
    # a block found inside another segment, at another offset: position-independent
    b, p = ix.lookup(_toks(4, 9) + t[4:8] + t[0:4] + [1, 2], 7)
    assert b == [-1, 1, 0] and p == [-1, 104, 100]
    # partial tail block is never looked up
    assert ix.lookup(t[:7], 7) == ([0], [100])
    # unfrozen block with entries: freed at reference count 0, entries gone
    u = ix.alloc(2)
    assert u == [3, 4]
    ix.insert(_toks(6, 2), 5, u, 0, frozen=False)            # one full block + partial
    assert ix.stats()[3] == 4
    ix.release(u)
    assert ix.stats() == (3, 7, 3, 3)


def test_eviction_order_and_threshold():
    """Above 90% in use, unheld frozen blocks go, fewest hits first, then
    the earliest frozen."""
    ix = si.BlockIndex(10, 2)
    segs = []
    for s in range(4):                            # 4 frozen blocks, one per segment
        b = ix.alloc(1)
        t = _toks(2, 10 + s)
        ix.insert(t, 1, b, 0, frozen=True)
        ix.release(b)
        segs.append((b[0], t))
    # hits: block 0 -> 2, block 1 -> 0, block 2 -> 1, block 3 -> 0
    for blk, t in (segs[0], segs[0], segs[2]):
        got, _ = ix.lookup(t, 1)
        assert got == [blk]
        ix.release(got)
    held = ix.alloc(5)                            # 9 of 10 in use: not above 90%
    assert held == [4, 5, 6, 7, 8] and ix.stats()[2] == 4
    ix.alloc(1)                                   # 10 in use -> evict one: block 1 (0 hits, frozen first)
    assert ix.stats() == (9, 1, 3, 3) and not ix.used[1]
    assert ix.lookup(segs[1][1], 1) == ([-1], [-1])
    ix.alloc(1)                                   # takes the freed block 1, then evicts block 3
    assert not ix.used[3] and ix.used[1] and ix.stats() == (9, 1, 2, 2)
    ix.alloc(1)                                   # next: block 2 (1 hit) before block 0 (2 hits)
    assert not ix.used[2] and ix.used[0]


def test_held_frozen_blocks_are_not_evicted_and_failed_alloc_changes_nothing():
    ix = si.BlockIndex(4, 2, evict_num=1, evict_den=2)
    b = ix.alloc(2)
    t = _toks(4, 3)
    ix.insert(t, 0, b, 0, frozen=True)            # held (ref 1) and frozen
    before = (list(ix.used), list(ix.ref), list(ix.frozen), len(ix.entries))
    with pytest.raises(MemoryError):
        ix.alloc(3)
    assert (list(ix.used), list(ix.ref), list(ix.frozen), len(ix.entries)) == before
    assert ix.alloc(2) == [2, 3]                  # 100% in use, nothing evictable
    ix.release(b)
    ix.release([2])                               # frees block 2 only: eviction runs in alloc
    assert ix.stats() == (3, 1, 2, 2)
    assert ix.alloc(1) == [2]                     # 4 in use -> evict both frozen (0 hits, 0 first)
    assert ix.stats() == (2, 2, 0, 0)


def test_most_recent_entry_wins_and_remove_api():
    ix = si.BlockIndex(8, 2)
    t = _toks(2, 4)
    a = ix.alloc(1)
    ix.insert(t, 3, a, 40, frozen=True)
    b = ix.alloc(1)
    ix.insert(t, 3, b, 90, frozen=True)          # same content cached twice
    assert ix.lookup(t, 3) == (b, [90])
    ix.remove(b)                                  # delete from the frozen pool; still held
    assert ix.used[b[0]] and not ix.frozen[b[0]]
    assert ix.lookup(t, 3) == (a, [40])
    ix.release(b + b)                             # insert's and the lookup's references
    assert not ix.used[b[0]]
    with pytest.raises(ValueError):
        ix.release(b)


def test_hash_collision_is_not_a_match(monkeypatch):
    monkeypatch.setattr(si, "virtual_hash", lambda tokens, key: 42)
    ix = si.BlockIndex(4, 2)
    a = ix.alloc(2)
    ix.insert([1, 2, 3, 4], 0, a, 0, frozen=True)
    assert ix.lookup([3, 4, 1, 2], 0) == (a[::-1], [2, 0])
    assert ix.lookup([1, 3, 2, 4], 0) == ([-1, -1], [-1, -1])


def test_plan_segments_hand_case():
    # blocks: hit 7@32, hit 8@36 (continues), miss, hit 3@0, hit 9@200 (jump), partial 3 tokens
    segs, ids, pieces = si.plan_segments(1, 100, [7, 8, -1, 3, 9], [32, 36, -1, 0, 200], 4, 23,
                                         ids_off=5)
    assert ids == [7, 8, 3, 9]
    assert segs == [dict(req=1, dst_start=100, len=8, p_src=32, src_slot0=0, src_pages_off=5),
                    dict(req=1, dst_start=112, len=4, p_src=0, src_slot0=0, src_pages_off=7),
                    dict(req=1, dst_start=116, len=4, p_src=200, src_slot0=0, src_pages_off=8)]
    assert pieces == [("reuse", 8), ("new", 4), ("reuse", 8), ("new", 3)]
    assert si.plan_segments(0, 0, [], [], 16, 5) == ([], [], [("new", 5)])


def test_random_sequences_keep_the_pool_consistent():
    """Invariants over random operation sequences: used + free = n; a free
    block has no entries, no references and is not frozen; every entry's
    block is in use; every lookup hit returns the token ids it was asked
    for (checked against the inserted segments, a plain list scan)."""
    rng = random.Random(7)
    for trial in range(30):
        ix = si.BlockIndex(24, 4, evict_num=rng.randint(5, 10), evict_den=10)
        held, cached = [], []          # cached: (tokens, key, block_ids, p_src)
        for _ in range(60):
            op = rng.random()
            try:
                if op < 0.3:
                    n = rng.randint(1, 6)
                    ids = ix.alloc(n)
                    toks = [rng.randint(0, 5) for _ in range(n * 4 - rng.randint(0, 3))]
                    key = rng.randint(0, 2)
                    ix.insert(toks, key, ids, rng.randint(0, 50), frozen=rng.random() < 0.7)
                    cached.append((toks, key, ids))
                    held.extend(ids)
                elif op < 0.55 and held:
                    k = rng.randrange(len(held))
                    ix.release([held.pop(k)])
                elif op < 0.85 and cached:
                    toks, key, _ = rng.choice(cached)
                    blocks, _ = ix.lookup(toks, key)
                    for j, b in enumerate(blocks):
                        if b >= 0:
                            e = [x for x in ix.entries if x["block"] == b]
                            assert any(x["tokens"] == tuple(toks[4 * j:4 * j + 4]) and x["key"] == key
                                       for x in e)
                            held.append(b)
                elif held:
                    b = rng.choice(held)
                    if ix.used[b]:
                        ix.remove([b])
            except MemoryError:
                pass
            used = sum(ix.used)
            assert ix.stats()[0] + ix.stats()[1] == 24 and ix.stats()[0] == used
            for b in range(24):
                if not ix.used[b]:
                    assert ix.ref[b] == 0 and not ix.frozen[b]
                    assert all(e["block"] != b for e in ix.entries)
                else:
                    assert ix.ref[b] > 0 or ix.frozen[b]
            assert sorted(held) == sorted(b for b in range(24) for _ in range(ix.ref[b]))
