// Segment lookup: the host-side index that maps a reused segment's token ids
// and extra key to cached KV blocks ("SparseX: Efficient Segment-Level KV
// Cache Sharing for Interleaved LLM Serving", §4.1 frozen blocks, §4.2 the
// frozen-block pool, §4.3 extra keys and h_virt = H(B, e), §4.4 virtual
// blocks, §4.5 block retrieval).  Pure host code; no GPU call is made here.
//
// Data structures, sized for pools of up to a few million blocks:
//   - per block: in-use flag, reference count, frozen flag, hit count and
//     the clock value at which it was frozen;
//   - free blocks in an ordered set (allocation takes the lowest ids);
//   - evictable blocks (frozen, reference count 0) in an ordered set keyed
//     by (hits, frozen-at, id), so the least-referenced one is its first;
//   - virtual entries in a slab with a hash multimap h_virt -> entry and a
//     per-block list of its entries.  A hit compares the extra key and the
//     stored token ids, so a 64-bit hash collision never matches.
#include <cstdint>
#include <cstring>
#include <set>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "sx.h"
#include "sx_internal.hpp"

using namespace sx;

namespace {

#define SX_REQUIRE(cond, code, ...)                  \
  do {                                               \
    if (!(cond)) return set_error(code, __VA_ARGS__); \
  } while (0)

// ---------------------------------------------------------------------------
// SHA-256 (FIPS 180-4).  The round constants are the first 32 fraction bits
// of the cube roots of the first 64 primes and the initial value those of
// the square roots of the first 8 primes (FIPS 180-4 §4.2.2, §5.3.3); they
// are derived here from that definition with exact integer roots.
// ---------------------------------------------------------------------------

using u128 = unsigned __int128;

// floor(p^(1/r) * 2^32) for r = 2 or 3: the largest x with x^r <= p * 2^(32 r).
uint64_t iroot_scaled(uint64_t p, int r) {
  const u128 target = (u128)p << (32 * r);
  uint64_t lo = 0, hi = (uint64_t)1 << 40;   // p < 2^9: the root is < 2^35
  while (lo < hi) {
    const uint64_t mid = lo + (hi - lo + 1) / 2;
    u128 pw = 1;
    for (int i = 0; i < r; ++i) pw *= mid;
    if (pw <= target) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

struct Sha256Consts {
  uint32_t k[64];
  uint32_t h0[8];
  Sha256Consts() {
    int n = 0;
    for (uint64_t c = 2; n < 64; ++c) {
      bool prime = true;
      for (uint64_t d = 2; d * d <= c; ++d)
        if (c % d == 0) { prime = false; break; }
      if (!prime) continue;
      k[n] = (uint32_t)iroot_scaled(c, 3);   // keeps the low 32 bits: the fraction
      if (n < 8) h0[n] = (uint32_t)iroot_scaled(c, 2);
      ++n;
    }
  }
};

const Sha256Consts& sha_consts() {
  static const Sha256Consts c;
  return c;
}

inline uint32_t rotr(uint32_t x, int s) { return (x >> s) | (x << (32 - s)); }

void sha256_block(uint32_t h[8], const uint8_t* p) {
  const Sha256Consts& C = sha_consts();
  uint32_t w[64];
  for (int t = 0; t < 16; ++t)
    w[t] = (uint32_t)p[4 * t] << 24 | (uint32_t)p[4 * t + 1] << 16 | (uint32_t)p[4 * t + 2] << 8 |
           (uint32_t)p[4 * t + 3];
  for (int t = 16; t < 64; ++t) {
    const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
    const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
    w[t] = w[t - 16] + s0 + w[t - 7] + s1;
  }
  uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
  for (int t = 0; t < 64; ++t) {
    const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = hh + S1 + ch + C.k[t] + w[t];
    const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
    const uint32_t t2 = S0 + maj;
    hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
  }
  h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
}

void sha256(const uint8_t* msg, size_t len, uint8_t out[32]) {
  uint32_t h[8];
  memcpy(h, sha_consts().h0, sizeof(h));
  size_t off = 0;
  for (; off + 64 <= len; off += 64) sha256_block(h, msg + off);
  // tail: the rest of the message, 0x80, zeros, the 64-bit big-endian bit length
  uint8_t tail[128] = {0};
  const size_t rest = len - off;
  memcpy(tail, msg + off, rest);
  tail[rest] = 0x80;
  const size_t tl = rest + 9 <= 64 ? 64 : 128;
  const uint64_t bits = (uint64_t)len * 8;
  for (int i = 0; i < 8; ++i) tail[tl - 1 - i] = (uint8_t)(bits >> (8 * i));
  sha256_block(h, tail);
  if (tl == 128) sha256_block(h, tail + 64);
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j) out[4 * i + j] = (uint8_t)(h[i] >> (24 - 8 * j));
}

// h_virt = H(B, e): SHA-256 of (e as 8 little-endian bytes, then each token
// id as 4 little-endian bytes); the first 8 digest bytes, little endian.
uint64_t virtual_hash(const int32_t* tok, int n, uint64_t key) {
  uint8_t small[8 + 4 * 64];
  std::vector<uint8_t> big;
  uint8_t* m = small;
  if (n > 64) {
    big.resize(8 + 4 * (size_t)n);
    m = big.data();
  }
  for (int i = 0; i < 8; ++i) m[i] = (uint8_t)(key >> (8 * i));
  for (int t = 0; t < n; ++t) {
    const uint32_t u = (uint32_t)tok[t];
    for (int i = 0; i < 4; ++i) m[8 + 4 * (size_t)t + i] = (uint8_t)(u >> (8 * i));
  }
  uint8_t d[32];
  sha256(m, 8 + 4 * (size_t)n, d);
  uint64_t h = 0;
  for (int i = 0; i < 8; ++i) h |= (uint64_t)d[i] << (8 * i);
  return h;
}

}  // namespace

// ---------------------------------------------------------------------------
// The index
// ---------------------------------------------------------------------------

struct sx_index {
  int32_t n, bs, num, den;
  int64_t clock = 0;
  int32_t n_used = 0, n_frozen = 0, n_live = 0;
  std::vector<uint8_t> used, frozen;
  std::vector<int32_t> ref;
  std::vector<int64_t> hits, frozen_at;
  std::set<int32_t> free_ids;
  std::set<std::tuple<int64_t, int64_t, int32_t>> evictable;   // (hits, frozen_at, id)
  // virtual entries
  std::vector<uint64_t> e_hash, e_key;
  std::vector<int32_t> e_block, e_pos;
  std::vector<int64_t> e_seq;
  std::vector<int32_t> e_tok;          // bs token ids per entry
  std::vector<int32_t> e_free;         // recycled entry slots
  std::unordered_multimap<uint64_t, int32_t> by_hash;
  std::vector<std::vector<int32_t>> block_entries;

  bool is_evictable(int32_t b) const { return frozen[b] && ref[b] == 0; }
  std::tuple<int64_t, int64_t, int32_t> ekey(int32_t b) const { return {hits[b], frozen_at[b], b}; }
  // Every change of (frozen, ref, hits, frozen_at) of block b is bracketed by
  // unlist(b) ... relist(b) so the evictable set stays exact.
  void unlist(int32_t b) {
    if (is_evictable(b)) evictable.erase(ekey(b));
  }
  void relist(int32_t b) {
    if (is_evictable(b)) evictable.insert(ekey(b));
  }

  void drop_entries(int32_t b) {
    for (int32_t e : block_entries[b]) {
      auto range = by_hash.equal_range(e_hash[e]);
      for (auto it = range.first; it != range.second; ++it)
        if (it->second == e) { by_hash.erase(it); break; }
      e_block[e] = -1;
      e_free.push_back(e);
      --n_live;
    }
    block_entries[b].clear();
  }
  void free_block(int32_t b) {   // caller has unlisted b
    drop_entries(b);
    if (frozen[b]) --n_frozen;
    used[b] = 0; frozen[b] = 0; ref[b] = 0; hits[b] = 0;
    free_ids.insert(b);
    --n_used;
  }
  bool evict_one() {
    if (evictable.empty()) return false;
    const int32_t b = std::get<2>(*evictable.begin());
    evictable.erase(evictable.begin());
    free_block(b);
    return true;
  }
};

extern "C" {

sx_status sx_virtual_hash(const int32_t* tokens_h, int32_t n_tok, uint64_t extra_key,
                          uint64_t* hash_h) {
  SX_REQUIRE(hash_h && (tokens_h || n_tok == 0), SX_EINVAL, "sx_virtual_hash: NULL argument");
  SX_REQUIRE(n_tok >= 0, SX_EINVAL, "sx_virtual_hash: n_tok < 0");
  *hash_h = virtual_hash(tokens_h, n_tok, extra_key);
  return SX_OK;
}

sx_status sx_index_create(int32_t n_blocks, int32_t block_size, int32_t evict_num,
                          int32_t evict_den, sx_index** index_h) {
  SX_REQUIRE(index_h, SX_EINVAL, "sx_index_create: index_h is NULL");
  *index_h = nullptr;
  SX_REQUIRE(n_blocks > 0 && block_size > 0, SX_EINVAL,
             "sx_index_create: n_blocks and block_size must be positive");
  SX_REQUIRE(evict_den > 0 && evict_num >= 0 && evict_num <= evict_den, SX_EINVAL,
             "sx_index_create: eviction threshold must be a fraction in [0, 1]");
  sx_index* ix = new sx_index();
  ix->n = n_blocks; ix->bs = block_size; ix->num = evict_num; ix->den = evict_den;
  ix->used.assign(n_blocks, 0);
  ix->frozen.assign(n_blocks, 0);
  ix->ref.assign(n_blocks, 0);
  ix->hits.assign(n_blocks, 0);
  ix->frozen_at.assign(n_blocks, 0);
  ix->block_entries.resize(n_blocks);
  for (int32_t b = 0; b < n_blocks; ++b) ix->free_ids.insert(ix->free_ids.end(), b);
  *index_h = ix;
  return SX_OK;
}

void sx_index_destroy(sx_index* index) { delete index; }

sx_status sx_index_alloc(sx_index* ix, int32_t n, int32_t* ids_h) {
  SX_REQUIRE(ix && (ids_h || n == 0), SX_EINVAL, "sx_index_alloc: NULL argument");
  SX_REQUIRE(n >= 0, SX_EINVAL, "sx_index_alloc: n < 0");
  SX_REQUIRE((int64_t)ix->free_ids.size() + (int64_t)ix->evictable.size() >= n, SX_ENOMEM,
             "sx_index_alloc: %d blocks requested, %zu free and %zu evictable", n,
             ix->free_ids.size(), ix->evictable.size());
  while ((int64_t)ix->free_ids.size() < n) ix->evict_one();
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = *ix->free_ids.begin();
    ix->free_ids.erase(ix->free_ids.begin());
    ix->used[b] = 1; ix->ref[b] = 1; ix->hits[b] = 0;
    ++ix->n_used;
    ids_h[i] = b;
  }
  while ((int64_t)ix->n_used * ix->den > (int64_t)ix->num * ix->n && ix->evict_one()) {
  }
  return SX_OK;
}

sx_status sx_index_release(sx_index* ix, const int32_t* ids_h, int32_t n) {
  SX_REQUIRE(ix && (ids_h || n == 0), SX_EINVAL, "sx_index_release: NULL argument");
  SX_REQUIRE(n >= 0, SX_EINVAL, "sx_index_release: n < 0");
  std::unordered_map<int32_t, int32_t> count;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = ids_h[i];
    SX_REQUIRE(b >= 0 && b < ix->n && ix->used[b], SX_EINVAL, "sx_index_release: block %d not in use", b);
    SX_REQUIRE(++count[b] <= ix->ref[b], SX_EINVAL,
               "sx_index_release: block %d released more often than it is held", b);
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = ids_h[i];
    ix->unlist(b);
    --ix->ref[b];
    if (ix->ref[b] == 0 && !ix->frozen[b]) ix->free_block(b);
    else ix->relist(b);
  }
  return SX_OK;
}

sx_status sx_index_insert(sx_index* ix, const int32_t* tokens_h, int32_t n_tok, uint64_t extra_key,
                          const int32_t* ids_h, int32_t p_src, int32_t frozen) {
  SX_REQUIRE(ix && (n_tok == 0 || (tokens_h && ids_h)), SX_EINVAL, "sx_index_insert: NULL argument");
  SX_REQUIRE(n_tok >= 0 && p_src >= 0, SX_EINVAL, "sx_index_insert: negative n_tok or p_src");
  const int32_t bs = ix->bs;
  const int32_t nb_all = (int32_t)(((int64_t)n_tok + bs - 1) / bs);
  for (int32_t j = 0; j < nb_all; ++j)
    SX_REQUIRE(ids_h[j] >= 0 && ids_h[j] < ix->n && ix->used[ids_h[j]], SX_EINVAL,
               "sx_index_insert: block %d not in use", ids_h[j]);
  for (int32_t j = 0; j < n_tok / bs; ++j) {
    const int32_t b = ids_h[j];
    int32_t e;
    if (!ix->e_free.empty()) {
      e = ix->e_free.back();
      ix->e_free.pop_back();
    } else {
      e = (int32_t)ix->e_block.size();
      ix->e_hash.push_back(0); ix->e_key.push_back(0); ix->e_block.push_back(-1);
      ix->e_pos.push_back(0); ix->e_seq.push_back(0);
      ix->e_tok.resize(ix->e_tok.size() + bs);
    }
    const int32_t* blk = tokens_h + (size_t)j * bs;
    ix->e_hash[e] = virtual_hash(blk, bs, extra_key);
    ix->e_key[e] = extra_key;
    ix->e_block[e] = b;
    ix->e_pos[e] = p_src + j * bs;
    ix->e_seq[e] = ++ix->clock;
    memcpy(&ix->e_tok[(size_t)e * bs], blk, sizeof(int32_t) * bs);
    ix->by_hash.emplace(ix->e_hash[e], e);
    ix->block_entries[b].push_back(e);
    ++ix->n_live;
    if (frozen && !ix->frozen[b]) {
      ix->unlist(b);
      ix->frozen[b] = 1;
      ix->frozen_at[b] = ++ix->clock;
      ++ix->n_frozen;
      ix->relist(b);
    }
  }
  return SX_OK;
}

sx_status sx_index_lookup(sx_index* ix, const int32_t* tokens_h, int32_t n_tok, uint64_t extra_key,
                          int32_t* block_h, int32_t* pos_h) {
  SX_REQUIRE(ix && (n_tok < ix->bs || (tokens_h && block_h && pos_h)), SX_EINVAL,
             "sx_index_lookup: NULL argument");
  SX_REQUIRE(n_tok >= 0, SX_EINVAL, "sx_index_lookup: n_tok < 0");
  const int32_t bs = ix->bs;
  for (int32_t j = 0; j < n_tok / bs; ++j) {
    const int32_t* blk = tokens_h + (size_t)j * bs;
    const uint64_t h = virtual_hash(blk, bs, extra_key);
    int32_t best = -1;
    auto range = ix->by_hash.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
      const int32_t e = it->second;
      if (ix->e_key[e] != extra_key) continue;
      if (memcmp(&ix->e_tok[(size_t)e * bs], blk, sizeof(int32_t) * bs) != 0) continue;
      if (best < 0 || ix->e_seq[e] > ix->e_seq[best]) best = e;
    }
    if (best < 0) {
      block_h[j] = -1;
      pos_h[j] = -1;
      continue;
    }
    const int32_t b = ix->e_block[best];
    ix->unlist(b);
    ++ix->ref[b];
    ++ix->hits[b];
    ix->relist(b);
    block_h[j] = b;
    pos_h[j] = ix->e_pos[best];
  }
  return SX_OK;
}

sx_status sx_index_remove(sx_index* ix, const int32_t* ids_h, int32_t n) {
  SX_REQUIRE(ix && (ids_h || n == 0), SX_EINVAL, "sx_index_remove: NULL argument");
  SX_REQUIRE(n >= 0, SX_EINVAL, "sx_index_remove: n < 0");
  for (int32_t i = 0; i < n; ++i)
    SX_REQUIRE(ids_h[i] >= 0 && ids_h[i] < ix->n && ix->used[ids_h[i]], SX_EINVAL,
               "sx_index_remove: block %d not in use", ids_h[i]);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = ids_h[i];
    if (!ix->used[b]) continue;   // listed twice, freed by its first mention
    ix->unlist(b);
    ix->drop_entries(b);
    if (ix->frozen[b]) --ix->n_frozen;
    ix->frozen[b] = 0;
    if (ix->ref[b] == 0) ix->free_block(b);
    else ix->relist(b);
  }
  return SX_OK;
}

sx_status sx_index_stats(const sx_index* ix, int32_t* stats_h) {
  SX_REQUIRE(ix && stats_h, SX_EINVAL, "sx_index_stats: NULL argument");
  stats_h[0] = ix->n_used;
  stats_h[1] = ix->n - ix->n_used;
  stats_h[2] = ix->n_frozen;
  stats_h[3] = ix->n_live;
  return SX_OK;
}

sx_status sx_plan_segments(int32_t req, int32_t dst_start, const int32_t* block_h,
                           const int32_t* pos_h, int32_t n_tok, int32_t block_size,
                           int32_t ids_off, sx_segment* segs_h, int32_t* n_segs_h,
                           int32_t* src_ids_h, int32_t* n_ids_h, int32_t* piece_reuse_h,
                           int32_t* piece_len_h, int32_t* n_pieces_h) {
  SX_REQUIRE(n_segs_h && n_ids_h && n_pieces_h && segs_h && src_ids_h && piece_reuse_h && piece_len_h,
             SX_EINVAL, "sx_plan_segments: NULL argument");
  SX_REQUIRE(block_size > 0 && n_tok >= 0 && req >= 0 && dst_start >= 0 && ids_off >= 0, SX_EINVAL,
             "sx_plan_segments: negative size or offset");
  const int32_t nb = n_tok / block_size;
  SX_REQUIRE(nb == 0 || (block_h && pos_h), SX_EINVAL, "sx_plan_segments: NULL lookup result");
  int32_t ns = 0, ni = 0, np = 0;
  auto add_piece = [&](int32_t reuse, int32_t L) {
    if (L <= 0) return;
    if (np > 0 && piece_reuse_h[np - 1] == reuse) {
      piece_len_h[np - 1] += L;
    } else {
      piece_reuse_h[np] = reuse;
      piece_len_h[np] = L;
      ++np;
    }
  };
  int32_t j = 0;
  while (j < nb) {
    if (block_h[j] < 0) {
      add_piece(0, block_size);
      ++j;
      continue;
    }
    const int32_t j0 = j;
    while (j + 1 < nb && block_h[j + 1] >= 0 && pos_h[j + 1] == pos_h[j] + block_size) ++j;
    ++j;
    sx_segment& s = segs_h[ns++];
    s.req = req;
    s.dst_start = dst_start + j0 * block_size;
    s.len = (j - j0) * block_size;
    s.p_src = pos_h[j0];
    s.src_slot0 = 0;
    s.src_pages_off = ids_off + ni;
    for (int32_t t = j0; t < j; ++t) src_ids_h[ni++] = block_h[t];
    add_piece(1, (j - j0) * block_size);
  }
  add_piece(0, n_tok - nb * block_size);
  *n_segs_h = ns;
  *n_ids_h = ni;
  *n_pieces_h = np;
  return SX_OK;
}

}  // extern "C"
