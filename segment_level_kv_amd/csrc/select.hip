// Sparse-Q key-token estimation and per-request top-k (SparseX paper §3.2:
// the probe of cost O(|I_nr| T d) and the paragraph after it -- one global
// per-token score aggregated across heads; §3.3 first sentence: globally
// important top-k tokens per request).
//
//   score[j] = sum_h sum_{i in I_nr, i >= j} exp(q_i^h . k_j / sqrt(d) - lse_i^h)
//
// Score pass (bf16): one workgroup per (256-key tile of a request, kv head)
// taking the G query heads of the group in turn, or, when that grid would
// leave compute units idle (short prompts), per (tile, query head); each
// wave keeps the K operand of its 64 keys in registers, the Sparse-Q rows
// stream through LDS two 32-row blocks per stage, S = Q . K^T runs on
// v_mfma_f32_32x32x16_bf16 with the key axis across lanes, and each lane
// sums exp(S - lse) over the queries in registers.  The MFMAs of the next
// block are issued before the exponentials of the current one, so the
// matrix cores and the VALU overlap inside each wave; the causal mask is
// applied only in blocks whose first row precedes the wave's last key.
// Partial sums per workgroup row go to a [parts][n_tok] buffer
// (parts = Hkv or Hq); the top-k adds them in row order, so every score is
// the same fixed-order fp32 sum run to run.
//
// Top-k: a multi-workgroup radix select over order-preserving 32-bit keys
// of the scores (-0 mapped to +0) with three digits and per-request global
// histograms, then per-chunk counts and an ordered compaction: all keys
// above the k-th largest plus the lowest-indexed keys equal to it, output
// ascending by token id.  Integer atomics only, so the result does not
// depend on the order workgroups run in.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "sx_device.hpp"
#include "sx_internal.hpp"

namespace sx {

namespace {

constexpr int SKT = 256;        // keys per score workgroup (4 waves x 64)
constexpr int SQB = 32;         // Sparse-Q rows per block (one MFMA row tile)
constexpr int SBS = 2;          // blocks per LDS stage
constexpr int SQP = 128 + 8;    // LDS row pitch in bf16 elements (16-byte pad: conflict-free b128 reads)

// Q rows are read when a block's MFMAs are issued, the normalisers and
// positions one block later (with its exponentials), hence three buffers
// for those.
struct ScoreSmem {
  uint16_t q[2][SBS * SQB][SQP];   // two stages of SBS blocks
  float lse2[3][SBS * SQB];        // log2-domain normaliser of each row (+inf: no row)
  int32_t qpos[3][SBS * SQB];      // row position in its request (INT_MAX: no row)
};

// Tile t of the score grid -> (request, first key index).  Tiles are laid
// out request by request, ceil(len / SKT) each.
__device__ __forceinline__ bool score_tile(const int32_t* seq_start, int n_req, int t, int& req,
                                           int& k0) {
  for (int r = 0; r < n_req; ++r) {
    const int len = seq_start[r + 1] - seq_start[r];
    const int nt = (len + SKT - 1) / SKT;
    if (t < nt) {
      req = r;
      k0 = t * SKT;
      return true;
    }
    t -= nt;
  }
  return false;
}

// One Sparse-Q block in flight: S = Q_blk . K^T for the wave's two 32-key
// columns.
struct ScoreBlock {
  f32x16 s[2];
};

// Sparse-Q row i of the batch into the score pass's layout: its q rows
// (q[q_index[i]], all heads) copied to q_g[i], its normalisers
// lse[lse_index[i]] times log2(e) to lse2_g[h][i] (head-major, so a block's
// 32 rows are one 128-byte line), and its position in its request to
// pos_g[i].  One workgroup per row.
__global__ __launch_bounds__(256) void sq_gather(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ q_index,
    const float* __restrict__ lse, const int32_t* __restrict__ lse_index,
    const int32_t* __restrict__ sq_rows, const int32_t* __restrict__ sq_start,
    const int32_t* __restrict__ seq_start, int n_req, int n_sq, int hq, uint16_t* __restrict__ q_g,
    float* __restrict__ lse2_g, int32_t* __restrict__ pos_g) {
  const int i = blockIdx.x, tid = threadIdx.x;
  const int qr = q_index ? q_index[i] : i;
  const u32x4* src = reinterpret_cast<const u32x4*>(q + (size_t)qr * hq * 128);
  u32x4* dst = reinterpret_cast<u32x4*>(q_g + (size_t)i * hq * 128);
  for (int c = tid; c < hq * 16; c += 256) dst[c] = src[c];
  if (tid < hq) {
    const int lr = lse_index ? lse_index[i] : i;
    lse2_g[(size_t)tid * n_sq + i] = lse[(size_t)lr * hq + tid] * kLog2e;
  }
  if (tid == 0) {
    // the request owning row i: the last r < n_req with sq_start[r] <= i
    int lo = 0, hi = n_req;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sq_start[mid] <= i) lo = mid;
      else hi = mid;
    }
    pos_g[i] = sq_rows[i] - seq_start[lo];
  }
}

// Sparse-Q rows in the score pass's layout (sq_gather above): row i of the
// batch's Sparse-Q list at q_g[i][h][:], its normalisers times log2(e) at
// lse2_g[h][i] and its position in its request at pos_g[i].
__global__ __launch_bounds__(256) void scores_bf16(
    const uint16_t* __restrict__ q_g, const float* __restrict__ lse2_g,
    const int32_t* __restrict__ pos_g, const int32_t* __restrict__ sq_start, sx_layout lay,
    int n_pages, const uint16_t* __restrict__ kpool, int hq, int hkv,
    float* __restrict__ partial, float scale_log2, int hpw, int n_sq) {
  __shared__ ScoreSmem sm;
  int req, k0;
  if (!score_tile(lay.seq_start, lay.n_req, blockIdx.x, req, k0)) return;
  const int G = hq / hkv;
  const int h0 = blockIdx.y * hpw;            // the hpw query heads of this workgroup
  const int g = h0 / G;                       // their kv head
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hl = lane >> 5;
  const int seq0 = lay.seq_start[req];
  const int len = lay.seq_start[req + 1] - seq0;
  const int32_t* bt = lay.block_table + (size_t)req * lay.max_pages;

  // K operand (B of S = Q K^T): this wave's keys k0 + 64w + 32nb + lane%32.
  bf16x8 kf[2][8];
  int key_idx[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int key = k0 + 64 * w + 32 * nb + (lane & 31);
    key_idx[nb] = key;
    const uint16_t* kp = nullptr;
    if (key < len && key / kPage < lay.max_pages) {
      const int page = bt[key / kPage];
      if (page >= 0 && page < n_pages)
        kp = kpool + (((size_t)page * hkv + g) * kPage + (key & (kPage - 1))) * 128 + hl * 8;
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 raw = kp ? *reinterpret_cast<const u32x4*>(kp + kk * 16) : u32x4{0, 0, 0, 0};
      kf[nb][kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const int kmax_w = k0 + 64 * w + 63;        // largest key of the wave

  // The Sparse-Q blocks that reach this key tile, head by head: block it is
  // rows bfirst + 32 (it % n_blk) .. of head h0 + it / n_blk.  Sparse-Q rows
  // are ascending, so the blocks wholly before the tile form a prefix that is
  // skipped.  Stage st (LDS buffer st & 1) holds blocks 2st and 2st + 1.
  const int s0 = sq_start[req], s1 = sq_start[req + 1];
  int bfirst = s0;
  while (bfirst < s1 && pos_g[min(bfirst + SQB, s1) - 1] < k0) bfirst += SQB;
  const int n_blk = (s1 - bfirst + SQB - 1) / SQB;
  const int n_it = n_blk * hpw;
  const int n_st = (n_it + SBS - 1) / SBS;
  constexpr int QU = SBS * SQB * 16 / 256;    // 16-byte Q chunks per thread and stage
  // Loads of stage st go to registers one stage ahead of their LDS store.
  // They are unconditional: an absent row reads row s0 of head h0, whose
  // finite q values are harmless because the row's normaliser is stored as
  // +inf (every exponential of the row is 0).  A load under a branch would
  // make the wait-count analysis drain every load in flight at the join.
  u32x4 qn[QU];
  float lse_n = 0.f;
  int pos_n = 0;
  bool okl = false;             // row tid (< SBS * SQB) exists
  int ix_b = 0, ix_h = h0;      // block-in-head and head of the next stage's first block
  const int lrow = tid & (SBS * SQB - 1);
  auto fetch = [&](int st) __attribute__((always_inline)) {
    int bb[SBS], hh[SBS];
#pragma unroll
    for (int k = 0; k < SBS; ++k) {
      const bool real = SBS * st + k < n_it;
      bb[k] = real ? ix_b : 0;
      hh[k] = real ? ix_h : h0;
      if (++ix_b == n_blk) {
        ix_b = 0;
        ++ix_h;
      }
    }
#pragma unroll
    for (int e = 0; e < QU; ++e) {
      const int u = tid + 256 * e;
      const int row = u >> 4, blk = row >> 5;
      const int i = bfirst + bb[blk] * SQB + (row & 31);
      const int ic = (SBS * st + blk < n_it && i < s1) ? i : s0;
      qn[e] = *reinterpret_cast<const u32x4*>(q_g + ((size_t)ic * hq + hh[blk]) * 128 + (u & 15) * 8);
    }
    const int blk = lrow >> 5;
    const int i = bfirst + bb[blk] * SQB + (lrow & 31);
    okl = tid < SBS * SQB && SBS * st + blk < n_it && i < s1;
    const int ic = okl ? i : s0;
    lse_n = lse2_g[(size_t)hh[blk] * n_sq + ic];
    pos_n = pos_g[ic];
  };
  auto stage_store = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < QU; ++e) {
      const int u = tid + 256 * e;
      *reinterpret_cast<u32x4*>(&sm.q[st & 1][u >> 4][(u & 15) * 8]) = qn[e];
    }
    if (tid < SBS * SQB) {
      sm.lse2[st % 3][tid] = okl ? lse_n : INFINITY;
      sm.qpos[st % 3][tid] = okl ? pos_n : INT_MAX;
    }
  };
  // S of block it; its Q rows are read from LDS here.
  auto issue = [&](int it, ScoreBlock& b) __attribute__((always_inline)) {
    const uint16_t* qr = &sm.q[(it / SBS) & 1][(it % SBS) * SQB + (lane & 31)][hl * 8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(qr + kk * 16);
      b.s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[0][kk], kk ? b.s[0] : f32x16{}, 0, 0, 0);
      b.s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[1][kk], kk ? b.s[1] : f32x16{}, 0, 0, 0);
    }
  };
  // Four accumulators per key column, added in a fixed order at the end.
  float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // Causal mask (row position >= key): only a block whose first row
  // precedes the wave's last key needs it (rows are ascending; the test is
  // wave-uniform).
  auto needs_mask = [&](int it) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(sm.qpos[(it / SBS) % 3][(it % SBS) * SQB]) <
           __builtin_amdgcn_readfirstlane(kmax_w);
  };
  // The exponentials of block itA (S in a) and, when ISSUE, the MFMAs of
  // block itB (into b) interleaved in one straight-line region, so each
  // wave keeps its matrix core and its VALU busy at the same time: two
  // MFMAs per eight-byte step of the head dimension, four of the 32
  // exponentials of the lane after each.
  auto step = [&](auto mask_c, auto issue_c, int itA, const ScoreBlock& a, int itB,
                  ScoreBlock& b) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value, ISSUE = decltype(issue_c)::value;
    const int bufA = (itA / SBS) % 3, rbA = (itA % SBS) * SQB;
    // accumulator register v of lane half hl holds block row 8(v>>2)+4hl+(v&3)
    float l[16];
    int qp[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[bufA][rbA + 8 * q4 + 4 * hl]);
#pragma unroll
      for (int e = 0; e < 4; ++e) l[4 * q4 + e] = l4[e];
      if (MASK) {
        const u32x4 p4 = *reinterpret_cast<const u32x4*>(&sm.qpos[bufA][rbA + 8 * q4 + 4 * hl]);
#pragma unroll
        for (int e = 0; e < 4; ++e) qp[4 * q4 + e] = (int)p4[e];
      }
    }
    const uint16_t* qr = &sm.q[(itB / SBS) & 1][(itB % SBS) * SQB + (lane & 31)][hl * 8];
    // v_exp_f32 directly: the argument is a log2 probability (<= 0 up to
    // rounding); below 2^-126 the term is below any score tolerance.
    auto elem = [&](int e) __attribute__((always_inline)) {
      const int nb = e >> 4, v = e & 15;
      float p = __builtin_amdgcn_exp2f(fmaf(a.s[nb][v], scale_log2, -l[v]));
      if (MASK) p = qp[v] >= key_idx[nb] ? p : 0.f;
      acc[nb][v & 3] += p;
    };
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      if (ISSUE) {
        const bf16x8 q8 = *reinterpret_cast<const bf16x8*>(qr + kk * 16);
        b.s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q8, kf[0][kk], kk ? b.s[0] : f32x16{}, 0, 0, 0);
        elem(4 * kk);
        elem(4 * kk + 1);
        b.s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q8, kf[1][kk], kk ? b.s[1] : f32x16{}, 0, 0, 0);
        elem(4 * kk + 2);
        elem(4 * kk + 3);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) elem(4 * kk + e);
      }
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto step_issue = [&](int itA, const ScoreBlock& a, int itB, ScoreBlock& b) __attribute__((always_inline)) {
    if (needs_mask(itA)) step(T_{}, T_{}, itA, a, itB, b);
    else step(F_{}, T_{}, itA, a, itB, b);
  };
  auto step_last = [&](int itA, const ScoreBlock& a) __attribute__((always_inline)) {
    ScoreBlock none;
    if (needs_mask(itA)) step(T_{}, F_{}, itA, a, itA, none);
    else step(F_{}, F_{}, itA, a, itA, none);
  };

  if (n_it > 0) {
    fetch(0);
    stage_store(0);
    __syncthreads();
    if (n_st > 1) fetch(1);
    ScoreBlock A, B;
    issue(0, A);
    // Software pipeline: block it+1's MFMAs run with block it's
    // exponentials.  Block it+1 may lie past the last block (odd n_it): its
    // MFMAs then read a stage buffer's stale rows and are never consumed.
    for (int it = 0; it < n_it; it += 2) {
      step_issue(it, A, it + 1, B);
      if (it + 2 < n_it) {
        if ((it + 2) % SBS == 0) {
          // Stage st's Q buffer was last read by the MFMAs of stage st - 2
          // and its normaliser buffer by the exponentials of stage st - 3;
          // every wave finished both before the previous barrier.
          const int st = (it + 2) / SBS;
          stage_store(st);
          __syncthreads();
          if (st + 1 < n_st) fetch(st + 1);
        }
        step_issue(it + 1, B, it + 2, A);
      } else if (it + 1 < n_it) {
        step_last(it + 1, B);
      }
    }
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float own = (acc[nb][0] + acc[nb][1]) + (acc[nb][2] + acc[nb][3]);
    const float tot = own + __shfl_xor(own, 32);
    if (hl == 0 && key_idx[nb] < len) partial[(size_t)blockIdx.y * lay.n_tok + seq0 + key_idx[nb]] = tot;
  }
}

// fp32 storage: one thread per (kv head, key); loops over the Sparse-Q rows
// and the query heads of the group in order.
template <int D>
__global__ __launch_bounds__(256) void scores_f32(
    const float* __restrict__ q, const int32_t* __restrict__ q_index,
    const int32_t* __restrict__ sq_rows, const int32_t* __restrict__ sq_start,
    const float* __restrict__ lse, const int32_t* __restrict__ lse_index, sx_layout lay,
    int n_pages, const float* __restrict__ kpool, int hq, int hkv, float* __restrict__ partial,
    float scale) {
  const int tok = blockIdx.x * blockDim.x + threadIdx.x;
  const int g = blockIdx.y;
  if (tok >= lay.n_tok) return;
  const int r = find_request(lay.seq_start, lay.n_req, tok);
  if (r < 0) return;
  const int seq0 = lay.seq_start[r];
  const int j = tok - seq0;
  const int page = page_of(lay, n_pages, r, j);
  const int G = hq / hkv;
  float sum = 0.f;
  if (page >= 0) {
    const float* kp = kpool + (((size_t)page * hkv + g) * kPage + (j & (kPage - 1))) * D;
    for (int i = sq_start[r]; i < sq_start[r + 1]; ++i) {
      if (sq_rows[i] - seq0 < j) continue;
      const int qr = q_index ? q_index[i] : i;
      const int lr = lse_index ? lse_index[i] : i;
      for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        const float* qp = q + ((size_t)qr * hq + h) * D;
        float dot = 0.f;
        for (int e = 0; e < D; ++e) dot = fmaf(qp[e], kp[e], dot);
        sum += expf(dot * scale - lse[(size_t)lr * hq + h]);
      }
    }
  }
  partial[(size_t)g * lay.n_tok + tok] = sum;
}

// ---------------------------------------------------------------------------
// Top-k
// ---------------------------------------------------------------------------
//
// Each request's tokens are cut into chunks of TK_CHUNK; every kernel below
// runs one workgroup per chunk.  Candidates are ordered by a 32-bit key
// (order_key of the score); the k-th largest key is found by a radix select
// over three digits (key bits 31-21, 20-10, 9-0): pass p counts, per
// request, the digits of the keys that share the digits already chosen,
// in a global histogram (integer atomics, so the counts do not depend on
// the order the workgroups run in), and every workgroup of the next kernel
// reads the histograms and picks the digit itself.  Then each chunk counts
// its keys above / equal to the threshold, and the last kernel places each
// chunk's selected tokens after those of the chunks before it (ties at the
// threshold go to the lowest token ids), in ascending token order.

constexpr int TK_THREADS = 256;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_PER = 4;                        // consecutive tokens per thread
constexpr int TK_CHUNK = TK_THREADS * TK_PER;    // tokens per workgroup
constexpr int TK_BINS0 = 2048, TK_BINS1 = 2048, TK_BINS2 = 1024;

// Per-request record in the workspace.
struct TopkReq {
  uint32_t hist0[TK_BINS0];    // key bits 31-21 of the candidates
  uint32_t hist1[TK_BINS1];    // bits 20-10 of the candidates matching the chosen bits 31-21
  uint32_t hist2[TK_BINS2];    // bits 9-0 of those matching bits 31-10
  int32_t n_cand;
  int32_t pad[63];
};
// Per-chunk counts: keys above the threshold, keys equal to it, class-1 tokens.
struct TopkChunk {
  int32_t gt, eq, c1, pad;
};

struct TkSmem {
  uint32_t hist[TK_BINS0];
  int32_t wsum[TK_WAVES];
  int32_t bcast[4];
};

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;                 // -0 == +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.
__device__ int tk_scan(int v, TkSmem& sm, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sm.wsum[w] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < TK_WAVES; ++i) {
    const int s = sm.wsum[i];
    before += (i < w) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Chunk c of the grid -> request and the grid index of the request's first
// chunk.  Chunks are laid out request by request, ceil(len / TK_CHUNK) each.
__device__ __forceinline__ bool tk_chunk(const int32_t* seq_start, int n_req, int c, int& req,
                                         int& first) {
  int base = 0;
  for (int r = 0; r < n_req; ++r) {
    const int nc = (seq_start[r + 1] - seq_start[r] + TK_CHUNK - 1) / TK_CHUNK;
    if (c < base + nc) {
      req = r;
      first = base;
      return true;
    }
    base += nc;
  }
  return false;
}

// The digit holding the want-th largest key (1 <= want <= the histogram's
// total) and the key's rank among the keys with that digit.  Thread t looks
// at bins NB-1-PER*t down to NB-PER*(t+1), so thread order is descending
// digit order.
template <int NB>
__device__ void tk_pick(const uint32_t* __restrict__ hist, int want, TkSmem& sm, uint32_t* digit,
                        int* rem) {
  constexpr int PER = NB / TK_THREADS;
  const int tid = threadIdx.x;
  int c[PER];
  int s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = (int)hist[NB - 1 - PER * tid - i];
    s += c[i];
  }
  int tot;
  const int above = tk_scan(s, sm, &tot);
  if (above < want && want <= above + s) {
    int cum = above;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (cum < want && want <= cum + c[i]) {
        sm.bcast[0] = NB - 1 - PER * tid - i;
        sm.bcast[1] = want - cum;
      }
      cum += c[i];
    }
  }
  __syncthreads();
  *digit = (uint32_t)sm.bcast[0];
  *rem = sm.bcast[1];
  __syncthreads();
}

// The key bits fixed by the first n_pass passes, their mask, and the rank
// (1-based) of the k-th largest key among the keys that carry them.
__device__ void tk_prefix(const TopkReq& st, int k, int n_pass, TkSmem& sm, uint32_t* prefix,
                          uint32_t* mask, int* rem) {
  uint32_t pf = 0, mk = 0, d;
  int want = k;
  if (n_pass > 0) {
    tk_pick<TK_BINS0>(st.hist0, want, sm, &d, &want);
    pf |= d << 21;
    mk |= 0x7ffu << 21;
  }
  if (n_pass > 1) {
    tk_pick<TK_BINS1>(st.hist1, want, sm, &d, &want);
    pf |= d << 10;
    mk |= 0x7ffu << 10;
  }
  if (n_pass > 2) {
    tk_pick<TK_BINS2>(st.hist2, want, sm, &d, &want);
    pf |= d;
    mk |= 0x3ffu;
  }
  *prefix = pf;
  *mask = mk;
  *rem = want;
}

__device__ __forceinline__ int tk_budget(const int32_t* k_sel, const TopkReq& st, int r) {
  return min(max(k_sel[r], 0), st.n_cand);
}

// Clears the per-request records.  A request with no tokens gets its padded
// outputs here (no chunk of it exists).
__global__ __launch_bounds__(TK_THREADS) void tk_init(TopkReq* __restrict__ st, int n_req,
                                                      const int32_t* __restrict__ seq_start,
                                                      const int32_t* __restrict__ k_sel,
                                                      const int32_t* __restrict__ sq_start,
                                                      int32_t* __restrict__ sel_rows,
                                                      int32_t* __restrict__ act_rows) {
  const int r = blockIdx.x;
  uint32_t* wd = reinterpret_cast<uint32_t*>(&st[r]);
  for (int i = threadIdx.x; i < (int)(sizeof(TopkReq) / 4); i += TK_THREADS) wd[i] = 0u;
  if (seq_start[r + 1] > seq_start[r]) return;
  int sel_off = 0;
  for (int i = 0; i < r; ++i) sel_off += max(k_sel[i], 0);
  const int k_req = max(k_sel[r], 0);
  for (int i = threadIdx.x; i < k_req; i += TK_THREADS) {
    sel_rows[sel_off + i] = -1;
    if (act_rows) act_rows[sq_start[r] + sel_off + i] = -1;
  }
}

// Pass 0: the scores (fixed-order sum of the partial rows), the candidate
// count and the histogram of key bits 31-21.
__global__ __launch_bounds__(TK_THREADS) void tk_pass0(
    const float* __restrict__ partial, int n_parts, int n_tok, const uint8_t* __restrict__ tok_class,
    const int32_t* __restrict__ seq_start, int n_req, const int32_t* __restrict__ k_sel,
    float* __restrict__ scores, TopkReq* __restrict__ st) {
  __shared__ TkSmem sm;
  int r, first;
  if (!tk_chunk(seq_start, n_req, blockIdx.x, r, first)) return;
  const int tid = threadIdx.x;
  const int t1 = seq_start[r + 1];
  const int j0 = seq_start[r] + (blockIdx.x - first) * TK_CHUNK + TK_PER * tid;
  const bool sum = n_parts > 1 || scores != partial;
  float sc[TK_PER];
  int cls[TK_PER];
#pragma unroll
  for (int u = 0; u < TK_PER; ++u) {
    const int j = j0 + u;
    cls[u] = j < t1 ? (int)tok_class[j] : 2;
    sc[u] = 0.f;
  }
  if (sum) {
    // eight partial rows loaded per round (unconditionally, at clamped
    // indices, so the loads are not serialised by branches), then added in
    // row order
    constexpr int PB = 8;
    for (int p0 = 0; p0 < n_parts; p0 += PB) {
      float v[PB][TK_PER];
#pragma unroll
      for (int p = 0; p < PB; ++p)
#pragma unroll
        for (int u = 0; u < TK_PER; ++u)
          v[p][u] = partial[(size_t)min(p0 + p, n_parts - 1) * n_tok + min(j0 + u, t1 - 1)];
#pragma unroll
      for (int p = 0; p < PB; ++p)
#pragma unroll
        for (int u = 0; u < TK_PER; ++u)
          if (p0 + p < n_parts) sc[u] += v[p][u];
    }
#pragma unroll
    for (int u = 0; u < TK_PER; ++u)
      if (j0 + u >= t1) sc[u] = 0.f;
#pragma unroll
    for (int u = 0; u < TK_PER; ++u)
      if (j0 + u < t1) scores[j0 + u] = sc[u];
  } else {
#pragma unroll
    for (int u = 0; u < TK_PER; ++u)
      if (j0 + u < t1) sc[u] = partial[j0 + u];
  }
  for (int i = tid; i < TK_BINS0; i += TK_THREADS) sm.hist[i] = 0u;
  __syncthreads();
  const bool need = k_sel[r] > 0;
  int cand = 0;
#pragma unroll
  for (int u = 0; u < TK_PER; ++u)
    if (cls[u] == 0) {
      ++cand;
      if (need) atomicAdd(&sm.hist[order_key(sc[u]) >> 21], 1u);
    }
  int n_cand;
  tk_scan(cand, sm, &n_cand);                  // also orders the LDS histogram updates
  if (tid == 0 && n_cand) atomicAdd(&st[r].n_cand, n_cand);
  if (need)
    for (int i = tid; i < TK_BINS0; i += TK_THREADS)
      if (sm.hist[i]) atomicAdd(&st[r].hist0[i], sm.hist[i]);
}

// Passes 1 and 2: histogram of key bits 20-10 (P = 1) or 9-0 (P = 2) of the
// candidates whose higher bits match the digits chosen so far.
template <int P>
__global__ __launch_bounds__(TK_THREADS) void tk_pass(const float* __restrict__ src,
                                                      const uint8_t* __restrict__ tok_class,
                                                      const int32_t* __restrict__ seq_start, int n_req,
                                                      const int32_t* __restrict__ k_sel,
                                                      TopkReq* __restrict__ st) {
  __shared__ TkSmem sm;
  int r, first;
  if (!tk_chunk(seq_start, n_req, blockIdx.x, r, first)) return;
  const int k = tk_budget(k_sel, st[r], r);
  if (k == 0) return;                          // uniform across the workgroup
  const int tid = threadIdx.x;
  const int t1 = seq_start[r + 1];
  const int j0 = seq_start[r] + (blockIdx.x - first) * TK_CHUNK + TK_PER * tid;
  uint32_t prefix, mask;
  int rem;
  tk_prefix(st[r], k, P, sm, &prefix, &mask, &rem);
  constexpr int NB = P == 1 ? TK_BINS1 : TK_BINS2;
  constexpr int SHIFT = P == 1 ? 10 : 0;
  for (int i = tid; i < NB; i += TK_THREADS) sm.hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < TK_PER; ++u) {
    const int j = j0 + u;
    if (j < t1 && tok_class[j] == 0) {
      const uint32_t key = order_key(src[j]);
      if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> SHIFT) & (NB - 1)], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = P == 1 ? st[r].hist1 : st[r].hist2;
  for (int i = tid; i < NB; i += TK_THREADS)
    if (sm.hist[i]) atomicAdd(&gh[i], sm.hist[i]);
}

// Per chunk: candidates above / equal to the k-th largest key, class-1 tokens.
__global__ __launch_bounds__(TK_THREADS) void tk_count(const float* __restrict__ src,
                                                       const uint8_t* __restrict__ tok_class,
                                                       const int32_t* __restrict__ seq_start, int n_req,
                                                       const int32_t* __restrict__ k_sel,
                                                       const TopkReq* __restrict__ st,
                                                       TopkChunk* __restrict__ cnt) {
  __shared__ TkSmem sm;
  int r, first;
  if (!tk_chunk(seq_start, n_req, blockIdx.x, r, first)) return;
  const int k = tk_budget(k_sel, st[r], r);
  const int tid = threadIdx.x;
  const int t1 = seq_start[r + 1];
  const int j0 = seq_start[r] + (blockIdx.x - first) * TK_CHUNK + TK_PER * tid;
  uint32_t thr = 0, mask = 0;
  int rem = 0;
  if (k > 0) tk_prefix(st[r], k, 3, sm, &thr, &mask, &rem);
  int ge = 0, n1 = 0;                           // gt | eq << 16 (each <= TK_CHUNK); class-1 count
#pragma unroll
  for (int u = 0; u < TK_PER; ++u) {
    const int j = j0 + u;
    if (j >= t1) continue;
    const int c = tok_class[j];
    n1 += c == 1;
    if (c == 0 && k > 0) {
      const uint32_t key = order_key(src[j]);
      ge += key > thr ? 1 : (key == thr ? 1 << 16 : 0);
    }
  }
  int ge_tot, n1_tot;
  tk_scan(ge, sm, &ge_tot);
  tk_scan(n1, sm, &n1_tot);
  if (tid == 0) cnt[blockIdx.x] = TopkChunk{ge_tot & 0xffff, ge_tot >> 16, n1_tot, 0};
}

// Ordered output: each chunk's selected tokens (and active rows) follow
// those of the request's earlier chunks.
__global__ __launch_bounds__(TK_THREADS) void tk_emit(
    const float* __restrict__ src, const uint8_t* __restrict__ tok_class,
    const int32_t* __restrict__ seq_start, int n_req, const int32_t* __restrict__ k_sel,
    const int32_t* __restrict__ sq_start, const TopkReq* __restrict__ st,
    const TopkChunk* __restrict__ cnt, int32_t* __restrict__ sel_rows, int32_t* __restrict__ act_rows) {
  __shared__ TkSmem sm;
  int r, first;
  if (!tk_chunk(seq_start, n_req, blockIdx.x, r, first)) return;
  const int k = tk_budget(k_sel, st[r], r);
  const int k_req = max(k_sel[r], 0);
  const int tid = threadIdx.x;
  const int t0 = seq_start[r], t1 = seq_start[r + 1];
  const int ci = blockIdx.x - first;
  const int j0 = t0 + ci * TK_CHUNK + TK_PER * tid;
  uint32_t thr = 0, mask = 0;
  int need_eq = 0;
  if (k > 0) tk_prefix(st[r], k, 3, sm, &thr, &mask, &need_eq);
  int sel_off = 0;
  for (int i = 0; i < r; ++i) sel_off += max(k_sel[i], 0);
  const int act_off = act_rows ? sq_start[r] + sel_off : 0;

  // Selected and active counts of the earlier chunks, in chunk order.
  int eq_before = 0, sel_before = 0, act_before = 0;
  for (int c0 = 0; c0 < ci; c0 += TK_THREADS) {
    const int c = c0 + tid;
    TopkChunk e = {0, 0, 0, 0};
    if (c < ci) e = cnt[first + c];
    int eq_tot;
    const int eq_ex = eq_before + tk_scan(e.eq, sm, &eq_tot);
    const int take_eq = min(max(need_eq - eq_ex, 0), e.eq);
    const int s = e.gt + take_eq;
    int s_tot, a_tot;
    tk_scan(s, sm, &s_tot);
    tk_scan(s + e.c1, sm, &a_tot);
    eq_before += eq_tot;
    sel_before += s_tot;
    act_before += a_tot;
  }

  // This chunk: flags of the thread's tokens, then two ordered scans.
  bool gt[TK_PER], eq[TK_PER], c1[TK_PER];
  int n_eq = 0;
#pragma unroll
  for (int u = 0; u < TK_PER; ++u) {
    const int j = j0 + u;
    const int c = j < t1 ? (int)tok_class[j] : 2;
    const uint32_t key = c == 0 ? order_key(src[j]) : 0u;
    gt[u] = c == 0 && k > 0 && key > thr;
    eq[u] = c == 0 && k > 0 && key == thr;
    c1[u] = c == 1;
    n_eq += eq[u];
  }
  int eq_tot;
  int eq_rank = eq_before + tk_scan(n_eq, sm, &eq_tot);
  bool sel[TK_PER];
  int n_sel = 0, n_act = 0;
#pragma unroll
  for (int u = 0; u < TK_PER; ++u) {
    sel[u] = gt[u] || (eq[u] && eq_rank < need_eq);
    eq_rank += eq[u];
    n_sel += sel[u];
    n_act += sel[u] || c1[u];
  }
  int pk_tot;
  const int pk = tk_scan(n_sel | (n_act << 16), sm, &pk_tot);
  int ps = sel_before + (pk & 0xffff), pa = act_before + (pk >> 16);
#pragma unroll
  for (int u = 0; u < TK_PER; ++u) {
    if (sel[u]) sel_rows[sel_off + ps++] = j0 + u;
    if (act_rows && (sel[u] || c1[u])) act_rows[act_off + pa++] = j0 + u;
  }
  // The request's last chunk pads budgets larger than the candidate count.
  const int n_chunks = (t1 - t0 + TK_CHUNK - 1) / TK_CHUNK;
  if (ci == n_chunks - 1) {
    const int act_total = act_before + (pk_tot >> 16);
    for (int i = k + tid; i < k_req; i += TK_THREADS) {
      sel_rows[sel_off + i] = -1;
      if (act_rows) act_rows[act_off + act_total + (i - k)] = -1;
    }
  }
}

}  // namespace

// Chunks of the top-k grid (>= the sum of the per-request chunk counts).
static int topk_chunks(int n_tok, int n_req) { return n_tok / TK_CHUNK + n_req + 1; }

size_t topk_ws_bytes(int n_tok, int n_req) {
  return align256((size_t)n_req * sizeof(TopkReq)) +
         align256((size_t)topk_chunks(n_tok, n_req) * sizeof(TopkChunk));
}

size_t select_ws_bytes(const sx_dims& d, int n_tok, int n_sq, int n_req) {
  return align256((size_t)score_parts(d, n_tok, n_req) * n_tok * sizeof(float))  // partial scores
         + align256((size_t)n_tok * sizeof(float))                // scores if caller passes none
         + align256((size_t)n_sq * d.n_q_heads * sizeof(float))   // probe LSE
         + std::max({attn_ws_bytes(d, n_sq, n_req, false),         // probe work list, then
                     scores_gather_bytes(d, n_sq),                 // the gathered Sparse-Q rows,
                     topk_ws_bytes(n_tok, n_req)});                // then the top-k records
}

// Key tiles of the score grid (>= the sum of the per-request tile counts).
int score_tiles(int n_tok, int n_req) { return n_tok / SKT + n_req + 1; }

// bf16: a workgroup takes the G query heads of one kv head, unless that grid
// would leave compute units idle (short prompts); then one query head each.
int score_parts(const sx_dims& d, int n_tok, int n_req) {
  if (d.dtype != SX_BF16) return d.n_kv_heads;
  return (long long)score_tiles(n_tok, n_req) * d.n_kv_heads < 512 ? d.n_q_heads : d.n_kv_heads;
}

size_t scores_gather_bytes(const sx_dims& d, int n_sq) {
  if (d.dtype != SX_BF16) return 0;
  return align256((size_t)n_sq * d.n_q_heads * 128 * sizeof(uint16_t)) +
         align256((size_t)n_sq * d.n_q_heads * sizeof(float)) + align256((size_t)n_sq * sizeof(int32_t));
}

sx_status launch_scores(const sx_dims& dims, const sx_layout& lay, const void* q,
                        const int32_t* q_index, const int32_t* sq_rows, const int32_t* sq_start,
                        int n_sq, const float* lse, const int32_t* lse_index,
                        const sx_pages& kv, float* partial, void* gather_ws, hipStream_t stream) {
  const int hq = dims.n_q_heads, hkv = dims.n_kv_heads, d = dims.head_dim;
  if (dims.dtype == SX_BF16) {
    char* p = static_cast<char*>(gather_ws);
    uint16_t* q_g = reinterpret_cast<uint16_t*>(p);
    p += align256((size_t)n_sq * hq * 128 * sizeof(uint16_t));
    float* lse2_g = reinterpret_cast<float*>(p);
    p += align256((size_t)n_sq * hq * sizeof(float));
    int32_t* pos_g = reinterpret_cast<int32_t*>(p);
    if (n_sq > 0) {
      sq_gather<<<n_sq, 256, 0, stream>>>((const uint16_t*)q, q_index, lse, lse_index, sq_rows, sq_start,
                                          lay.seq_start, lay.n_req, n_sq, hq, q_g, lse2_g, pos_g);
      const sx_status st = check_launch("sx_select_topk (Sparse-Q gather)");
      if (st != SX_OK) return st;
    }
    const int parts = score_parts(dims, lay.n_tok, lay.n_req);
    scores_bf16<<<dim3(score_tiles(lay.n_tok, lay.n_req), parts), 256, 0, stream>>>(
        q_g, lse2_g, pos_g, sq_start, lay, kv.n_pages, (const uint16_t*)kv.k, hq, hkv, partial,
        kLog2e / sqrtf((float)d), hq / parts, n_sq);
  } else {
    dim3 grid((lay.n_tok + 255) / 256, hkv);
    const float scale = 1.f / sqrtf((float)d);
    if (d == 64)
      scores_f32<64><<<grid, 256, 0, stream>>>((const float*)q, q_index, sq_rows, sq_start, lse,
                                                lse_index, lay, kv.n_pages, (const float*)kv.k,
                                                hq, hkv, partial, scale);
    else
      scores_f32<128><<<grid, 256, 0, stream>>>((const float*)q, q_index, sq_rows, sq_start, lse,
                                                 lse_index, lay, kv.n_pages, (const float*)kv.k,
                                                 hq, hkv, partial, scale);
  }
  return check_launch("sx_select_topk (scores)");
}

sx_status launch_topk(const float* partial, int n_parts, const uint8_t* tok_class,
                      const int32_t* seq_start, int n_req, int n_tok, const int32_t* k_sel,
                      const int32_t* sq_start, int32_t* sel_rows, int32_t* act_rows,
                      float* scores_out, void* ws, hipStream_t stream) {
  if (n_req == 0) return SX_OK;
  TopkReq* st = static_cast<TopkReq*>(ws);
  TopkChunk* cnt = reinterpret_cast<TopkChunk*>(static_cast<char*>(ws) +
                                                align256((size_t)n_req * sizeof(TopkReq)));
  const int nc = topk_chunks(n_tok, n_req);
  const float* src = (n_parts > 1 || scores_out != partial) ? scores_out : partial;
  tk_init<<<n_req, TK_THREADS, 0, stream>>>(st, n_req, seq_start, k_sel, sq_start, sel_rows, act_rows);
  tk_pass0<<<nc, TK_THREADS, 0, stream>>>(partial, n_parts, n_tok, tok_class, seq_start, n_req, k_sel,
                                           scores_out, st);
  tk_pass<1><<<nc, TK_THREADS, 0, stream>>>(src, tok_class, seq_start, n_req, k_sel, st);
  tk_pass<2><<<nc, TK_THREADS, 0, stream>>>(src, tok_class, seq_start, n_req, k_sel, st);
  tk_count<<<nc, TK_THREADS, 0, stream>>>(src, tok_class, seq_start, n_req, k_sel, st, cnt);
  tk_emit<<<nc, TK_THREADS, 0, stream>>>(src, tok_class, seq_start, n_req, k_sel, sq_start, st, cnt,
                                          sel_rows, act_rows);
  return check_launch("top-k");
}

}  // namespace sx
