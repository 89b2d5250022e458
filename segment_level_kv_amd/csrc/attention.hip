// Causal GQA attention of the active rows over the mixed paged KV cache
// (SparseX paper §3.2: Sparse-Q rows attend to all available keys at their
// true positions; §3.4: full attention before the threshold, Sparse-Q plus
// selected rows after it; §4.5 last paragraph: reused blocks are read through
// the block table, recomputed tokens take the normal attention path).
//
// bf16 kernel (gfx950): one workgroup = one query tile (64 consecutive
// active rows of one request) x one kv head; wave w owns query head
// g*G + w for all 64 rows, so the G heads sharing a kv head share every K/V
// block staged in LDS.  Per 64-key block:
//   S^T[key][q] = K . Q^T        (v_mfma_f32_32x32x16_bf16, Q in registers)
//   online softmax over the key axis, which sits in registers (16 keys per
//   lane per 32-key block; one cross-half exchange for the row max)
//   O^T[d][q] += V^T . P^T        (P^T straight from the S^T accumulators)
// Keys are permuted inside each 32-key block when K rows are loaded, so that
// the accumulator registers of S^T are exactly the B operand of the PV
// product (8 consecutive keys per lane half).  V pages are stored [d][slot],
// so the V^T operand is one contiguous 16-byte LDS read.  K/V blocks are
// double-buffered in LDS with register prefetch; only blocks that reach
// past the tile's first row apply the causal mask.
//
// Scheduling: tiles are ordered longest first (last tile of each request
// first), and workgroup b takes kv head b % Hkv so that with 8 kv heads each
// XCD streams a single head's K/V through its L2.
#include "sx_device.hpp"
#include "sx_internal.hpp"

namespace sx {

namespace {

constexpr int KB = 64;                 // keys per block
constexpr int LDK = 128 + 8;           // padded K row (bf16 elements)
constexpr int LDV = KB + 8;            // padded V^T row

template <int G>
struct AttnSmem {
  uint16_t k[2][KB][LDK];
  uint16_t v[2][128][LDV];
};

// Tile table: tiles of kTileRows rows per request; ordered by rank from the
// request's end (largest positions first), then by request.
// Rows outside [0, n_rows) (an inconsistent row_start) produce no tile, and
// at most max_tiles tiles are written.
__global__ __launch_bounds__(256) void build_tiles(const int32_t* __restrict__ row_start, int n_req,
                                                   int n_rows, int max_tiles,
                                                   AttnTile* __restrict__ tiles, int* __restrict__ n_tiles) {
  extern __shared__ int cnt[];
  for (int r = threadIdx.x; r < n_req; r += blockDim.x) {
    const int a = max(row_start[r], 0), b = min(row_start[r + 1], n_rows);
    const int n = b - a;
    cnt[r] = n > 0 ? (n + kTileRows - 1) / kTileRows : 0;
  }
  __syncthreads();
  int total = 0;
  for (int r = 0; r < n_req; ++r) total += cnt[r];
  if (threadIdx.x == 0) *n_tiles = min(total, max_tiles);
  for (int r = 0; r < n_req; ++r) {
    const int c = cnt[r];
    for (int t = threadIdx.x; t < c; t += blockDim.x) {
      int pos = 0;
      for (int r2 = 0; r2 < n_req; ++r2) pos += min(cnt[r2], t) + ((r2 < r && cnt[r2] > t) ? 1 : 0);
      if (pos >= max_tiles) continue;
      const int a = max(row_start[r], 0), b = min(row_start[r + 1], n_rows);
      const int row0 = a + (c - 1 - t) * kTileRows;
      AttnTile tl;
      tl.req = r;
      tl.row0 = row0;
      tl.nrows = min(kTileRows, b - row0);
      tl.pad = 0;
      tiles[pos] = tl;
    }
  }
}

template <int G, bool WITH_O>
__global__ __launch_bounds__(G * 64) void attn_bf16(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ q_index,
    const int32_t* __restrict__ rows, sx_layout lay, int n_pages,
    const uint16_t* __restrict__ kpool, const uint16_t* __restrict__ vpool, int hkv,
    uint16_t* __restrict__ o, float* __restrict__ lse, const AttnTile* __restrict__ tiles,
    const int* __restrict__ n_tiles, float scale_log2) {
  constexpr int NT = G * 64;
  constexpr int KU = (KB * 16 + NT - 1) / NT;      // 16-byte K units per thread per block
  constexpr int VU = (128 * 8 + NT - 1) / NT;      // 16-byte V units per thread per block
  extern __shared__ __align__(16) unsigned char smem_raw[];
  AttnSmem<G>& sm = *reinterpret_cast<AttnSmem<G>*>(smem_raw);

  const int g = blockIdx.x % hkv;
  const int ti = blockIdx.x / hkv;
  if (ti >= *n_tiles) return;
  const AttnTile tl = tiles[ti];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hq = G * hkv;
  const int h = g * G + w;
  const int req = tl.req;
  const int seq0 = lay.seq_start[req];
  const int seq_len = lay.seq_start[req + 1] - seq0;
  auto row_index = [&](int m) { return (rows ? rows[m] : m) - seq0; };
  const int p_min = row_index(tl.row0);
  const int p_max = row_index(tl.row0 + tl.nrows - 1);
  if (p_min < 0 || p_max >= seq_len || p_min > p_max) return;

  // ---- this lane's two queries (N-blocks of 32) ---------------------------
  const int hl = lane >> 5;           // lane half
  int pos_q[2];
  bf16x8 qf[2][8];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int qi = (lane & 31) + 32 * nb;
    const bool valid = qi < tl.nrows;
    const int m = tl.row0 + qi;
    pos_q[nb] = valid ? row_index(m) : p_max;
    const uint16_t* qp = q + ((size_t)(valid ? (q_index ? q_index[m] : m) : 0) * hq + h) * 128 + hl * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 raw = valid ? *reinterpret_cast<const u32x4*>(qp + kk * 16) : u32x4{0, 0, 0, 0};
      qf[nb][kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- K/V block loader ----------------------------------------------------
  const int32_t* bt = lay.block_table + (size_t)req * lay.max_pages;
  const int last_page = p_max / kPage;
  u32x4 rk[KU], rv[VU];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = tid + NT * i;
      rk[i] = u32x4{0, 0, 0, 0};
      if (u < KB * 16) {
        const int kl = u >> 4, c = u & 15;
        const int key = kb + kl;
        const int pi = key / kPage;
        if (key <= p_max && pi < lay.max_pages) {
          const int page = bt[pi];
          if (page >= 0 && page < n_pages)
            rk[i] = *reinterpret_cast<const u32x4*>(
                kpool + (((size_t)page * hkv + g) * kPage + (key & (kPage - 1))) * 128 + c * 8);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = tid + NT * i;
      rv[i] = u32x4{0, 0, 0, 0};
      if (u < 128 * 8) {
        const int d = u >> 3, c8 = u & 7;
        const int key0 = kb + c8 * 8;               // 8 keys of one page
        const int pi = key0 / kPage;
        if (pi <= last_page && pi < lay.max_pages) {
          const int page = bt[pi];
          if (page >= 0 && page < n_pages) {
            u32x4 raw = *reinterpret_cast<const u32x4*>(
                vpool + (((size_t)page * hkv + g) * 128 + d) * kPage + (key0 & (kPage - 1)));
            if (key0 + 7 > p_max) {                 // zero keys past the tile's last row
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (key0 + 2 * e > p_max) raw[e] &= 0u;
                else if (key0 + 2 * e + 1 > p_max) raw[e] &= 0xffffu;
              }
            }
            rv[i] = raw;
          }
        }
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = tid + NT * i;
      if (u < KB * 16) *reinterpret_cast<u32x4*>(&sm.k[buf][u >> 4][(u & 15) * 8]) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = tid + NT * i;
      if (u < 128 * 8) *reinterpret_cast<u32x4*>(&sm.v[buf][u >> 3][(u & 7) * 8]) = rv[i];
    }
  };

  // K row loaded by this lane for the S^T A-operand (key permutation inside
  // a 32-key block: accumulator register v of lane half hl then holds key
  // 16*(v>>3) + 8*hl + (v&7)).
  const int mrow = lane & 31;
  const int kperm = 16 * (mrow >> 4) + 8 * ((mrow >> 2) & 1) + 4 * ((mrow >> 3) & 1) + (mrow & 3);

  f32x16 oacc[4][2];
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) oacc[md][nb] = f32x16{};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  const int n_blk = p_max / KB + 1;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int b = 0; b < n_blk; ++b) {
    const int buf = b & 1;
    const int kb = b * KB;
    if (b + 1 < n_blk) gload(kb + KB);

    // S^T = K . Q^T for two 32-key M-blocks
    f32x16 s[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb][0] = f32x16{};
      s[mb][1] = f32x16{};
      const uint16_t* kr = &sm.k[buf][mb * 32 + kperm][hl * 8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + kk * 16);
        s[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[0][kk], s[mb][0], 0, 0, 0);
        s[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[1][kk], s[mb][1], 0, 0, 0);
      }
    }

    // online softmax (log2 domain)
    const bool need_mask = kb + KB - 1 > p_min;
    bf16x8 pb[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float t = s[mb][nb][v] * scale_log2;
          if (need_mask) {
            const int key = kb + 32 * mb + 16 * (v >> 3) + 8 * hl + (v & 7);
            t = key > pos_q[nb] ? -INFINITY : t;
          }
          s[mb][nb][v] = t;
          mx = fmaxf(mx, t);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[nb], mx);
      const float alpha = exp2f(m_run[nb] - m_new);
      m_run[nb] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
          float p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            p[i] = exp2f(s[mb][nb][hv * 8 + i] - m_new);
            ls += p[i];
          }
          u32x4 pk;
#pragma unroll
          for (int i = 0; i < 4; ++i) pk[i] = pack_bf2(p[2 * i], p[2 * i + 1]);
          pb[nb][mb * 2 + hv] = __builtin_bit_cast(bf16x8, pk);
        }
      l_run[nb] = l_run[nb] * alpha + ls;
      if (WITH_O) {
#pragma unroll
        for (int md = 0; md < 4; ++md) oacc[md][nb] *= alpha;
      }
    }

    if (WITH_O) {
      // O^T += V^T . P^T
#pragma unroll
      for (int md = 0; md < 4; ++md) {
        const uint16_t* vr = &sm.v[buf][md * 32 + (lane & 31)][hl * 8];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vr + ks * 16);
          oacc[md][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[0][ks], oacc[md][0], 0, 0, 0);
          oacc[md][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[1][ks], oacc[md][1], 0, 0, 0);
        }
      }
    }
    if (b + 1 < n_blk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue --------------------------------------------------------------
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int qi = (lane & 31) + 32 * nb;
    const bool valid = qi < tl.nrows;
    const float l_tot = l_run[nb] + __shfl_xor(l_run[nb], 32);
    const int m = tl.row0 + qi;
    if (lse && valid && hl == 0) lse[(size_t)m * hq + h] = (m_run[nb] + __log2f(l_tot)) * kLn2;
    if (WITH_O && valid) {
      const float inv = 1.f / l_tot;
      uint16_t* op = o + ((size_t)m * hq + h) * 128 + 4 * hl;
#pragma unroll
      for (int md = 0; md < 4; ++md)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 pk;
          pk[0] = pack_bf2(oacc[md][nb][4 * j] * inv, oacc[md][nb][4 * j + 1] * inv);
          pk[1] = pack_bf2(oacc[md][nb][4 * j + 2] * inv, oacc[md][nb][4 * j + 3] * inv);
          *reinterpret_cast<u32x2*>(op + md * 32 + 8 * j) = pk;
        }
    }
  }
}

// fp32 storage: one wave per (row, query head); lanes split the head
// dimension, keys are visited in order with an online softmax.
template <int D>
__global__ __launch_bounds__(64) void attn_rows_f32(
    const float* __restrict__ q, const int32_t* __restrict__ q_index,
    const int32_t* __restrict__ rows, int n_rows, sx_layout lay, int n_pages,
    const float* __restrict__ kpool, const float* __restrict__ vpool, int hkv, int hq,
    float* __restrict__ o, float* __restrict__ lse, float scale) {
  constexpr int E = D / 64;
  const int m = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int g = h / (hq / hkv);
  const int tok = rows ? rows[m] : m;
  const int r = find_request(lay.seq_start, lay.n_req, tok);
  if (r < 0) return;
  const int i = tok - lay.seq_start[r];
  const float* qp = q + ((size_t)(q_index ? q_index[m] : m) * hq + h) * D;
  float qv[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qv[e] = qp[lane + 64 * e];
    acc[e] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int j = 0; j <= i; ++j) {
    const int page = page_of(lay, n_pages, r, j);
    if (page < 0) continue;
    const float* kp = kpool + (((size_t)page * hkv + g) * kPage + (j & (kPage - 1))) * D;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) part = fmaf(qv[e], kp[lane + 64 * e], part);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    const float sc = part * scale;
    const float m_new = fmaxf(m_run, sc);
    const float alpha = expf(m_run - m_new);
    const float p = expf(sc - m_new);
    l_run = l_run * alpha + p;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float vv = vpool[(((size_t)page * hkv + g) * D + lane + 64 * e) * kPage + (j & (kPage - 1))];
      acc[e] = acc[e] * alpha + p * vv;
    }
    m_run = m_new;
  }
  if (o) {
#pragma unroll
    for (int e = 0; e < E; ++e) o[((size_t)m * hq + h) * D + lane + 64 * e] = acc[e] / l_run;
  }
  if (lse && lane == 0) lse[(size_t)m * hq + h] = m_run + logf(l_run);
}

template <int G, bool WITH_O>
sx_status launch_attn_bf16(int grid, const void* q, const int32_t* q_index, const int32_t* rows,
                      const sx_layout& lay, const sx_pages& kv, int hkv, void* o, float* lse,
                      const AttnTile* tiles, const int* n_tiles, float scale_log2,
                      hipStream_t stream) {
  const size_t smem = sizeof(AttnSmem<G>);
  const sx_status st = allow_lds((const void*)attn_bf16<G, WITH_O>, smem, "attention");
  if (st != SX_OK) return st;
  attn_bf16<G, WITH_O><<<grid, G * 64, smem, stream>>>(
      (const uint16_t*)q, q_index, rows, lay, kv.n_pages, (const uint16_t*)kv.k,
      (const uint16_t*)kv.v, hkv, (uint16_t*)o, lse, tiles, n_tiles, scale_log2);
  return SX_OK;
}

template <bool WITH_O>
sx_status dispatch_g(int G, int grid, const void* q, const int32_t* q_index, const int32_t* rows,
                     const sx_layout& lay, const sx_pages& kv, int hkv, void* o, float* lse,
                     const AttnTile* tiles, const int* n_tiles, float scale_log2, hipStream_t s) {
  switch (G) {
    case 1: return launch_attn_bf16<1, WITH_O>(grid, q, q_index, rows, lay, kv, hkv, o, lse, tiles, n_tiles, scale_log2, s);
    case 2: return launch_attn_bf16<2, WITH_O>(grid, q, q_index, rows, lay, kv, hkv, o, lse, tiles, n_tiles, scale_log2, s);
    case 4: return launch_attn_bf16<4, WITH_O>(grid, q, q_index, rows, lay, kv, hkv, o, lse, tiles, n_tiles, scale_log2, s);
    case 7: return launch_attn_bf16<7, WITH_O>(grid, q, q_index, rows, lay, kv, hkv, o, lse, tiles, n_tiles, scale_log2, s);
    case 8: return launch_attn_bf16<8, WITH_O>(grid, q, q_index, rows, lay, kv, hkv, o, lse, tiles, n_tiles, scale_log2, s);
    default: return set_error(SX_EUNSUPPORTED, "bf16 attention: n_q_heads/n_kv_heads = %d not built (1,2,4,7,8)", G);
  }
}

}  // namespace

size_t attn_ws_bytes(int n_rows, int n_req) {
  const size_t max_tiles = (size_t)(n_rows + kTileRows - 1) / kTileRows + (size_t)n_req;
  return align256(sizeof(int)) + align256(max_tiles * sizeof(AttnTile));
}

sx_status launch_attention(const sx_dims& dims, const sx_layout& lay, const void* q,
                           const int32_t* q_index, const int32_t* rows,
                           const int32_t* row_start, int n_rows, const sx_pages& kv, void* o,
                           float* lse, void* ws, hipStream_t stream) {
  if (n_rows == 0) return SX_OK;
  const int hq = dims.n_q_heads, hkv = dims.n_kv_heads, d = dims.head_dim;
  if (dims.dtype != SX_BF16) {
    const float scale = 1.f / sqrtf((float)d);
    dim3 grid(n_rows, hq);
    if (d == 64)
      attn_rows_f32<64><<<grid, 64, 0, stream>>>((const float*)q, q_index, rows, n_rows, lay,
                                                 kv.n_pages, (const float*)kv.k, (const float*)kv.v,
                                                 hkv, hq, (float*)o, lse, scale);
    else
      attn_rows_f32<128><<<grid, 64, 0, stream>>>((const float*)q, q_index, rows, n_rows, lay,
                                                  kv.n_pages, (const float*)kv.k, (const float*)kv.v,
                                                  hkv, hq, (float*)o, lse, scale);
    return check_launch("attention (fp32)");
  }
  int* n_tiles = reinterpret_cast<int*>(ws);
  AttnTile* tiles = reinterpret_cast<AttnTile*>(static_cast<char*>(ws) + align256(sizeof(int)));
  const int max_tiles = (n_rows + kTileRows - 1) / kTileRows + lay.n_req;
  build_tiles<<<1, 256, (size_t)lay.n_req * sizeof(int), stream>>>(row_start, lay.n_req, n_rows,
                                                                    max_tiles, tiles, n_tiles);
  sx_status st = check_launch("attention tile table");
  if (st != SX_OK) return st;
  const int G = hq / hkv;
  const float scale_log2 = kLog2e / sqrtf((float)d);
  const int grid = max_tiles * hkv;
  st = o ? dispatch_g<true>(G, grid, q, q_index, rows, lay, kv, hkv, o, lse, tiles, n_tiles, scale_log2, stream)
         : dispatch_g<false>(G, grid, q, q_index, rows, lay, kv, hkv, o, lse, tiles, n_tiles, scale_log2, stream);
  if (st != SX_OK) return st;
  return check_launch("attention");
}

}  // namespace sx
