"""Segment lookup over a shared block pool -- TEST INFRASTRUCTURE ONLY.

Plain-Python oracle of the host index that turns a reused segment's token
ids and extra key into block hits and realign descriptors.  Only ``tests/``
may import it; it shares no code with the library.

Source: "SparseX: Efficient Segment-Level KV Cache Sharing for Interleaved
LLM Serving", §4.1 (frozen blocks), §4.2 (frozen-block pool), §4.3 (extra
keys, the virtual hash h_virt = H(B, e)), §4.4 (virtual blocks) and §4.5
(block retrieval and reuse).  Where the sections leave a step open the
reading taken is stated at the method that takes it.

Everything is a linear scan over plain lists; the only library routine used
is hashlib's SHA-256 as the hash H.
"""

from __future__ import annotations

import hashlib


def virtual_hash(tokens, extra_key: int) -> int:
    """h_virt = H(B, e) of §4.3 for one block B of token ids and extra key e.

    Reading taken (the section names no hash function): H is SHA-256 over
    the 8-byte little-endian extra key followed by each token id as a 4-byte
    little-endian signed integer; h_virt is the first 8 digest bytes read as
    a little-endian unsigned 64-bit integer.  No parent hash is chained in:
    a virtual block is position- and prefix-independent (§4.4).
    """
    data = int(extra_key).to_bytes(8, "little", signed=False)
    for t in tokens:
        data += int(t).to_bytes(4, "little", signed=True)
    return int.from_bytes(hashlib.sha256(data).digest()[:8], "little")


class BlockIndex:
    """Block pool bookkeeping plus the virtual-block index (§4.1-§4.4).

    The pool has n_blocks physical blocks of block_size tokens.  Per block:
    in use or free, a reference count, a frozen flag, a hit count (lookups
    that returned it) and, once frozen, the order in which it was frozen.
    A virtual block (§4.4) is an index entry {h_virt, physical block,
    position of the block's first token in the cached copy, the block's
    token ids, extra key}; it owns no KV memory.

    Readings taken:
      - alloc(n) takes the n lowest free block ids, reference count 1.  If
        fewer than n are free it first evicts frozen blocks nobody holds;
        if even that cannot supply n it fails and changes nothing.  After
        allocating, while more than evict_num/evict_den of the pool is in
        use (§4.1: e.g. above 90% utilisation), it keeps evicting unheld
        frozen blocks.  "Least-referenced" (§4.1) is read as the fewest
        lookup hits; ties go to the block frozen earliest, then the lower
        id.
      - Evicting a frozen block drops its virtual entries and frees it.
      - Calls taking a list of ids check the whole list before changing
        anything, so a failed call leaves the index as it was.
      - release(ids) drops one reference per id; an unfrozen block whose
        count reaches 0 is freed and its virtual entries dropped (an
        ordinary block returns to the free list, §4.1); a frozen block stays.
      - insert registers one virtual entry per full block of a cached
        segment; frozen=True also freezes those blocks (§4.2 insert API).
        The partial last block of a segment gets no entry.
      - lookup hashes each full block, and among the live entries with that
        hash compares extra key and token ids (no false match on a hash
        collision, §4.3); of several matches the most recently inserted
        wins.  Each hit takes a reference on the block (the source must stay
        alive until the realign copy is done) and counts a hit.
      - remove(ids) is the §4.2 delete API: drops the blocks' entries and
        unfreezes them; a block nobody holds is freed.
    """

    def __init__(self, n_blocks: int, block_size: int, evict_num: int = 9, evict_den: int = 10):
        if n_blocks <= 0 or block_size <= 0 or evict_den <= 0 or not 0 <= evict_num <= evict_den:
            raise ValueError("bad pool parameters")
        self.n, self.bs = n_blocks, block_size
        self.num, self.den = evict_num, evict_den
        self.used = [False] * n_blocks
        self.ref = [0] * n_blocks
        self.frozen = [False] * n_blocks
        self.hits = [0] * n_blocks
        self.frozen_at = [0] * n_blocks
        self.entries = []          # dicts: h, block, pos, tokens, key, seq
        self.clock = 0

    # -- helpers ---------------------------------------------------------------
    def _tick(self) -> int:
        self.clock += 1
        return self.clock

    def _drop_entries(self, b: int):
        self.entries = [e for e in self.entries if e["block"] != b]

    def _free(self, b: int):
        self._drop_entries(b)
        self.used[b] = False
        self.frozen[b] = False
        self.ref[b] = 0
        self.hits[b] = 0

    def _evictable(self):
        return [b for b in range(self.n) if self.frozen[b] and self.ref[b] == 0]

    def _evict_one(self) -> bool:
        cand = self._evictable()
        if not cand:
            return False
        b = min(cand, key=lambda i: (self.hits[i], self.frozen_at[i], i))
        self._free(b)
        return True

    def n_used(self) -> int:
        return sum(self.used)

    # -- API -------------------------------------------------------------------
    def alloc(self, n: int) -> list:
        if n < 0:
            raise ValueError("n < 0")
        free = [b for b in range(self.n) if not self.used[b]]
        if len(free) + len(self._evictable()) < n:
            raise MemoryError("pool exhausted")
        while sum(not u for u in self.used) < n:
            self._evict_one()
        ids = [b for b in range(self.n) if not self.used[b]][:n]
        for b in ids:
            self.used[b] = True
            self.ref[b] = 1
            self.hits[b] = 0
        while self.n_used() * self.den > self.num * self.n and self._evict_one():
            pass
        return ids

    def release(self, ids):
        ids = [int(b) for b in ids]
        for b in ids:      # validate the whole list first: an error changes nothing
            if not (0 <= b < self.n) or not self.used[b] or ids.count(b) > self.ref[b]:
                raise ValueError(f"block {b} is not held that often")
        for b in ids:
            self.ref[b] -= 1
            if self.ref[b] == 0 and not self.frozen[b]:
                self._free(b)

    def insert(self, tokens, extra_key: int, block_ids, p_src: int, frozen: bool):
        tokens = [int(t) for t in tokens]
        nb_all = (len(tokens) + self.bs - 1) // self.bs
        if len(block_ids) != nb_all:
            raise ValueError("one block id per (partial) block")
        for b in block_ids:
            if not (0 <= b < self.n) or not self.used[b]:
                raise ValueError(f"block {b} is not in use")
        for j in range(len(tokens) // self.bs):
            blk = tokens[j * self.bs:(j + 1) * self.bs]
            b = int(block_ids[j])
            self.entries.append(dict(h=virtual_hash(blk, extra_key), block=b,
                                     pos=int(p_src) + j * self.bs, tokens=tuple(blk),
                                     key=int(extra_key), seq=self._tick()))
            if frozen and not self.frozen[b]:
                self.frozen[b] = True
                self.frozen_at[b] = self._tick()

    def lookup(self, tokens, extra_key: int):
        tokens = [int(t) for t in tokens]
        blocks, pos = [], []
        for j in range(len(tokens) // self.bs):
            blk = tuple(tokens[j * self.bs:(j + 1) * self.bs])
            h = virtual_hash(blk, extra_key)
            match = [e for e in self.entries
                     if e["h"] == h and e["key"] == int(extra_key) and e["tokens"] == blk]
            if match:
                e = max(match, key=lambda x: x["seq"])
                self.ref[e["block"]] += 1
                self.hits[e["block"]] += 1
                blocks.append(e["block"])
                pos.append(e["pos"])
            else:
                blocks.append(-1)
                pos.append(-1)
        return blocks, pos

    def remove(self, ids):
        ids = [int(b) for b in ids]
        for b in ids:      # validate the whole list first: an error changes nothing
            if not (0 <= b < self.n) or not self.used[b]:
                raise ValueError(f"block {b} is not in use")
        for b in ids:
            if not self.used[b]:
                continue   # listed twice and freed by its first mention
            self._drop_entries(b)
            self.frozen[b] = False
            if self.ref[b] == 0:
                self._free(b)

    def stats(self):
        """(blocks in use, free blocks, frozen blocks, live virtual entries)."""
        return (self.n_used(), self.n - self.n_used(), sum(self.frozen), len(self.entries))


def plan_segments(req: int, dst_start: int, blocks, pos, block_size: int, n_tok: int,
                  ids_off: int = 0):
    """Realign descriptors of one reused piece from its lookup (§4.5).

    The piece has n_tok tokens starting at token index dst_start of request
    req; blocks/pos are the lookup result of its full blocks.  A run of
    consecutive hits whose cached positions continue block after block
    (pos[b+1] = pos[b] + block_size) becomes one segment {req, dst_start,
    len, p_src, src_slot0 = 0, src_pages_off}; the hit blocks' ids, in
    order, form the source page-id array starting at ids_off.  Misses and
    the partial last block are tokens to prefill (§4.5: separated, they
    take part in prefill).  Returns (segments, src_ids, pieces) with pieces
    the piece's split into ("reuse", L) / ("new", L) runs in order.
    """
    segs, src_ids, pieces = [], [], []

    def add_piece(kind, L):
        if L <= 0:
            return
        if pieces and pieces[-1][0] == kind:
            pieces[-1] = (kind, pieces[-1][1] + L)
        else:
            pieces.append((kind, L))

    nb = len(blocks)
    j = 0
    while j < nb:
        if blocks[j] < 0:
            add_piece("new", block_size)
            j += 1
            continue
        j0 = j
        while j + 1 < nb and blocks[j + 1] >= 0 and pos[j + 1] == pos[j] + block_size:
            j += 1
        j += 1
        segs.append(dict(req=req, dst_start=dst_start + j0 * block_size,
                         len=(j - j0) * block_size, p_src=pos[j0], src_slot0=0,
                         src_pages_off=ids_off + len(src_ids)))
        src_ids.extend(blocks[j0:j])
        add_piece("reuse", (j - j0) * block_size)
    add_piece("new", n_tok - nb * block_size)
    return segs, src_ids, pieces
