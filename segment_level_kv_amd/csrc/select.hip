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
// wave keeps the K operand of its 64 keys in registers, the Sparse-Q rows of
// one query head stream through LDS 32 at a time, S = Q . K^T runs on
// v_mfma_f32_32x32x16_bf16 with the key axis across lanes, and each lane
// sums exp(S - lse) over the queries in registers.  Partial sums per
// workgroup row go to a [parts][n_tok] buffer (parts = Hkv or Hq); the top-k
// kernel adds them in row order, so every score is the same fixed-order fp32
// sum run to run.
//
// Top-k: one workgroup per request.  Order-preserving 32-bit keys of the
// scores (-0 mapped to +0), a 4-pass 8-bit radix select for the k-th largest
// key in LDS (per-wave histograms), then an in-order compaction sweep with
// block prefix sums: all keys above the threshold plus the lowest-indexed
// keys equal to it.  Output is ascending by token id.  Every sweep issues a
// batch of loads per thread before using them (one workgroup per request
// would otherwise pay a memory round trip per element).
#include "sx_device.hpp"
#include "sx_internal.hpp"

namespace sx {

namespace {

constexpr int SKT = 256;        // keys per score workgroup
constexpr int SQB = 32;         // Sparse-Q rows per LDS block

struct ScoreSmem {
  uint16_t q[SQB][128 + 8];
  float lse2[SQB];
  int32_t qpos[SQB];
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

__global__ __launch_bounds__(256) void scores_bf16(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ q_index,
    const int32_t* __restrict__ sq_rows, const int32_t* __restrict__ sq_start,
    const float* __restrict__ lse, const int32_t* __restrict__ lse_index, sx_layout lay,
    int n_pages, const uint16_t* __restrict__ kpool, int hq, int hkv,
    float* __restrict__ partial, float scale_log2, int hpw) {
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

  const int s0 = sq_start[req], s1 = sq_start[req + 1];
  float acc[2] = {0.f, 0.f};
  // The Sparse-Q blocks that reach this key tile, visited head by head; the
  // next block's Q rows, LSE and positions are loaded into registers while
  // the current block is in the MFMAs.  Sparse-Q rows are ascending, so the
  // blocks wholly before the tile form a prefix that is skipped.
  int bfirst = s0;
  while (bfirst < s1 && sq_rows[min(bfirst + SQB, s1) - 1] - seq0 < k0) bfirst += SQB;
  const int n_blk = (s1 - bfirst + SQB - 1) / SQB;
  const int n_it = n_blk * hpw;              // iteration it: head h0 + it / n_blk, block it % n_blk
  constexpr int QU = SQB * 16 / 256;         // 16-byte Q chunks per thread and block
  u32x4 qn[QU];
  float lse_n = INFINITY;
  int pos_n = -1;
  auto fetch = [&](int it) __attribute__((always_inline)) {
    const int h = h0 + it / n_blk;
    const int b0 = bfirst + (it % n_blk) * SQB;
#pragma unroll
    for (int e = 0; e < QU; ++e) {
      const int u = tid + 256 * e;
      const int r = u >> 4, c = u & 15;
      const int i = b0 + r;
      qn[e] = u32x4{0, 0, 0, 0};
      if (i < s1) {
        const int qr = q_index ? q_index[i] : i;
        qn[e] = *reinterpret_cast<const u32x4*>(q + ((size_t)qr * hq + h) * 128 + c * 8);
      }
    }
    if (tid < SQB) {
      const int i = b0 + tid;
      lse_n = INFINITY;
      pos_n = -1;
      if (i < s1) {
        const int lr = lse_index ? lse_index[i] : i;
        lse_n = lse[(size_t)lr * hq + h] * kLog2e;
        pos_n = sq_rows[i] - seq0;
      }
    }
  };
  if (n_it > 0) fetch(0);
  for (int it = 0; it < n_it; ++it) {
    {
      __syncthreads();                        // every wave is done with the previous block
#pragma unroll
      for (int e = 0; e < QU; ++e) {
        const int u = tid + 256 * e;
        *reinterpret_cast<u32x4*>(&sm.q[u >> 4][(u & 15) * 8]) = qn[e];
      }
      if (tid < SQB) {
        sm.lse2[tid] = lse_n;
        sm.qpos[tid] = pos_n;
      }
      __syncthreads();
      if (it + 1 < n_it) fetch(it + 1);
      f32x16 s[2] = {f32x16{}, f32x16{}};
      const uint16_t* qr = &sm.q[lane & 31][hl * 8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(qr + kk * 16);
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[0][kk], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[1][kk], s[1], 0, 0, 0);
      }
      // accumulator register v of lane half hl holds query row 8(v>>2)+4hl+(v&3)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int qr_ = 8 * (v >> 2) + 4 * hl + (v & 3);
          // v_exp_f32 directly: the argument is a log2 probability (<= 0 up to
          // rounding); below 2^-126 the term is below any score tolerance.
          const float p = __builtin_amdgcn_exp2f(s[nb][v] * scale_log2 - sm.lse2[qr_]);
          acc[nb] += (sm.qpos[qr_] >= key_idx[nb]) ? p : 0.f;
        }
    }
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float tot = acc[nb] + __shfl_xor(acc[nb], 32);
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

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_BATCH = 8;           // rounds of TK_THREADS tokens loaded together

struct TopkSmem {
  uint32_t hist[TK_WAVES][256];
  int32_t wsum[TK_WAVES];
  int32_t bcast[4];
};

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;                 // -0 == +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive prefix sum over the workgroup; *total receives the sum.
__device__ int block_scan(int v, TopkSmem& sm, int* total) {
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
  for (int i = 0; i < TK_WAVES; ++i) {
    const int s = sm.wsum[i];
    before += (i < w) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(
    const float* __restrict__ partial, int n_parts, int n_tok, const uint8_t* __restrict__ tok_class,
    const int32_t* __restrict__ seq_start, const int32_t* __restrict__ k_sel,
    const int32_t* __restrict__ sq_start, int32_t* __restrict__ sel_rows,
    int32_t* __restrict__ act_rows, float* __restrict__ scores) {
  __shared__ TopkSmem sm;
  const int r = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6;
  const int t0 = seq_start[r], t1 = seq_start[r + 1];
  int sel_off = 0;
  for (int i = 0; i < r; ++i) sel_off += max(k_sel[i], 0);
  const int k_req = max(k_sel[r], 0);

  // Every loop below visits the request's tokens in batches of TK_BATCH per
  // thread (token t0 + tid + TK_THREADS * (b + u)), issuing all the batch's
  // loads before using any of them: a single workgroup would otherwise pay
  // one memory round trip per element per thread.
  constexpr int U = TK_BATCH;
  const int n = t1 - t0;
  const int n_rounds = (n + TK_THREADS - 1) / TK_THREADS;

  // pass 0: scores (fixed-order sum of the partial rows) and candidate count
  const float* src = partial;
  if (n_parts > 1 || scores != partial) {
    for (int b = 0; b < n_rounds; b += U) {
      float acc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] = 0.f;
      for (int p = 0; p < n_parts; ++p) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = t0 + tid + TK_THREADS * (b + u);
          v[u] = j < t1 ? partial[(size_t)p * n_tok + j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] += v[u];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = t0 + tid + TK_THREADS * (b + u);
        if (j < t1) scores[j] = acc[u];
      }
    }
    src = scores;
    __threadfence_block();
    __syncthreads();
  }
  // key and class of the batch starting at round b (class 2 past the end)
  auto load_batch = [&](int b, uint32_t (&key)[U], int (&cls)[U]) __attribute__((always_inline)) {
    float sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = t0 + tid + TK_THREADS * (b + u);
      cls[u] = j < t1 ? (int)tok_class[j] : 2;
      sv[u] = j < t1 ? src[j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) key[u] = cls[u] == 0 ? order_key(sv[u]) : 0u;
  };
  int my_cand = 0;
  for (int b = 0; b < n_rounds; b += U) {
    uint32_t key[U];
    int cls[U];
    load_batch(b, key, cls);
#pragma unroll
    for (int u = 0; u < U; ++u) my_cand += cls[u] == 0;
  }
  int n_cand;
  block_scan(my_cand, sm, &n_cand);
  const int k = min(k_req, n_cand);

  // radix select of the k-th largest key
  uint32_t prefix = 0, pmask = 0;
  int remaining = k;
  if (k > 0) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < TK_WAVES * 256; i += TK_THREADS) (&sm.hist[0][0])[i] = 0;
      __syncthreads();
      for (int b = 0; b < n_rounds; b += U) {
        uint32_t key[U];
        int cls[U];
        load_batch(b, key, cls);
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (cls[u] == 0 && (key[u] & pmask) == prefix) atomicAdd(&sm.hist[w][(key[u] >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 256) {
        uint32_t s = 0;
        for (int i = 0; i < TK_WAVES; ++i) s += sm.hist[i][tid];
        sm.hist[0][tid] = s;
      }
      __syncthreads();
      if (tid == 0) {
        int cum = 0, dsel = 0;
        for (int d = 255; d >= 0; --d) {
          const int c = (int)sm.hist[0][d];
          if (cum + c >= remaining) { dsel = d; break; }
          cum += c;
        }
        sm.bcast[0] = dsel;
        sm.bcast[1] = remaining - cum;
      }
      __syncthreads();
      prefix |= (uint32_t)sm.bcast[0] << shift;
      pmask |= 0xffu << shift;
      remaining = sm.bcast[1];
      __syncthreads();
    }
  }
  const uint32_t thr = prefix;       // key of the k-th largest candidate
  const int need_eq = remaining;     // how many keys equal to thr to take

  // in-order compaction, one round of TK_THREADS tokens at a time (a batch
  // of rounds loaded together)
  const int act_off = act_rows ? sq_start[r] + sel_off : 0;
  int base_eq = 0, base_sel = 0, base_act = 0;
  for (int b = 0; b < n_rounds; b += U) {
    uint32_t key[U];
    int cls[U];
    load_batch(b, key, cls);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (b + u >= n_rounds) break;                 // uniform across the workgroup
      const int j = t0 + tid + TK_THREADS * (b + u);
      const bool cand = cls[u] == 0 && k > 0;
      const bool gt = cand && key[u] > thr;
      const bool eq = cand && key[u] == thr;
      int tot_eq;
      const int eq_rank = base_eq + block_scan(eq ? 1 : 0, sm, &tot_eq);
      const bool sel = gt || (eq && eq_rank < need_eq);
      const bool act = sel || cls[u] == 1;
      int tot_pk;
      const int pk = block_scan((sel ? 1 : 0) | (act ? 1 << 16 : 0), sm, &tot_pk);
      if (sel) sel_rows[sel_off + base_sel + (pk & 0xffff)] = j;
      if (act && act_rows) act_rows[act_off + base_act + (pk >> 16)] = j;
      base_eq += tot_eq;
      base_sel += tot_pk & 0xffff;
      base_act += tot_pk >> 16;
    }
  }
  // budgets larger than the candidate count: pad with -1
  for (int i = k + tid; i < k_req; i += TK_THREADS) sel_rows[sel_off + i] = -1;
  if (act_rows)
    for (int i = base_act + tid; i < base_act + (k_req - k); i += TK_THREADS) act_rows[act_off + i] = -1;
}

}  // namespace

size_t topk_ws_bytes(int n_tok, int n_req) {
  (void)n_req;
  return align256((size_t)n_tok * sizeof(float));
}

size_t select_ws_bytes(const sx_dims& d, int n_tok, int n_sq, int n_req) {
  return align256((size_t)score_parts(d, n_tok, n_req) * n_tok * sizeof(float))  // partial scores
         + align256((size_t)n_tok * sizeof(float))                // scores if caller passes none
         + align256((size_t)n_sq * d.n_q_heads * sizeof(float))   // probe LSE
         + attn_ws_bytes(d, n_sq, n_req, false);                   // probe work list
}

// Key tiles of the score grid (>= the sum of the per-request tile counts).
int score_tiles(int n_tok, int n_req) { return n_tok / SKT + n_req + 1; }

// bf16: a workgroup takes the G query heads of one kv head, unless that grid
// would leave compute units idle (short prompts); then one query head each.
int score_parts(const sx_dims& d, int n_tok, int n_req) {
  if (d.dtype != SX_BF16) return d.n_kv_heads;
  return (long long)score_tiles(n_tok, n_req) * d.n_kv_heads < 512 ? d.n_q_heads : d.n_kv_heads;
}

sx_status launch_scores(const sx_dims& dims, const sx_layout& lay, const void* q,
                        const int32_t* q_index, const int32_t* sq_rows, const int32_t* sq_start,
                        int n_sq, const float* lse, const int32_t* lse_index,
                        const sx_pages& kv, float* partial, hipStream_t stream) {
  (void)n_sq;
  const int hq = dims.n_q_heads, hkv = dims.n_kv_heads, d = dims.head_dim;
  if (dims.dtype == SX_BF16) {
    const int parts = score_parts(dims, lay.n_tok, lay.n_req);
    scores_bf16<<<dim3(score_tiles(lay.n_tok, lay.n_req), parts), 256, 0, stream>>>(
        (const uint16_t*)q, q_index, sq_rows, sq_start, lse, lse_index, lay, kv.n_pages,
        (const uint16_t*)kv.k, hq, hkv, partial, kLog2e / sqrtf((float)d), hq / parts);
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
  (void)ws;
  if (n_req == 0) return SX_OK;
  topk_kernel<<<n_req, TK_THREADS, 0, stream>>>(partial, n_parts, n_tok, tok_class, seq_start,
                                                k_sel, sq_start, sel_rows, act_rows, scores_out);
  return check_launch("top-k");
}

}  // namespace sx
