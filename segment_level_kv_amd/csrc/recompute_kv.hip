// Sparse-KV recomputation (SparseX paper §3.4: K/V of the Sparse-Q rows and
// the selected top-k rows are recomputed in the same forward pass; §4.5:
// recomputed tokens take the normal attention path).
//
//   [q | k | v] = x[rows] . W_qkv^T ;  q, k rotated by R_pos ;
//   k, v scattered into the request's pages, q written densely.
//
// bf16 path: MFMA GEMM (v_mfma_f32_32x32x16_bf16), 128x128 output tiles
// (one tile column = one head of 128, so both halves of every rotate-half
// pair are in the tile), K-step 64 staged through LDS with a double buffer
// and register prefetch.  Tiles are assigned XCD-contiguously (workgroup b
// runs on XCD b % 8) and grouped 4 row-tiles at a time so that concurrently
// running workgroups share W and X slices in their XCD's L2.  The epilogue
// stages the fp32 tile in LDS, applies RoPE with the fp64-built table,
// rounds to bf16 and writes 16-byte chunks (Q, K) or page columns (V).
#include "sx_device.hpp"
#include "sx_internal.hpp"

namespace sx {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8;          // padded LDS row (elements) against bank conflicts
constexpr int LDC = BN + 4;
constexpr int GROUP_M = 4;

struct GemmSmem {
  union {
    struct {
      uint16_t a[2][BM][LDK];
      uint16_t b[2][BN][LDK];
    } ab;
    float c[BM][LDC];
  };
  int32_t row_req[BM];
  int32_t row_idx[BM];
};

__global__ __launch_bounds__(256) void qkv_gemm_bf16(
    const uint16_t* __restrict__ x, int hidden, const int32_t* __restrict__ rows, int n_rows,
    const uint16_t* __restrict__ w, int head0, int n_tiles_m, int n_tiles_n, sx_layout lay,
    int n_pages, uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool,
    uint16_t* __restrict__ q_out, int hq, int hkv) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  GemmSmem& sm = *reinterpret_cast<GemmSmem*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile assignment: XCD-contiguous ranges, grouped along M ----------
  const int total = n_tiles_m * n_tiles_n;
  const int per_xcd = (total + 7) / 8;
  const int t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (t >= total) return;
  const int group = t / (GROUP_M * n_tiles_n);
  const int first_m = group * GROUP_M;
  const int gsz = min(n_tiles_m - first_m, GROUP_M);
  const int within = t % (GROUP_M * n_tiles_n);
  const int mt = first_m + within % gsz;
  const int nt = within / gsz;
  const int m0 = mt * BM;
  const int head = head0 + nt;                 // 0..hq-1: Q, then K heads, then V heads
  const uint16_t* wt = w + (size_t)head * 128 * hidden;

  // ---- per-row request / index ---------------------------------------------
  if (tid < BM) {
    int r = -1, idx = 0;
    if (m0 + tid < n_rows) {
      const int tok = rows[m0 + tid];
      r = find_request(lay.seq_start, lay.n_req, tok);
      if (r >= 0) idx = tok - lay.seq_start[r];
    }
    sm.row_req[tid] = r;
    sm.row_idx[tid] = idx;
  }

  // ---- global -> register loaders (4 x 16 B per thread for A and for B) ---
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
  int l_row[4], l_chunk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + 256 * i;
    l_row[i] = u >> 3;
    l_chunk[i] = u & 7;
    const int m = m0 + l_row[i];
    int tok = (m < n_rows) ? rows[m] : -1;
    if (tok < 0 || tok >= lay.n_tok) tok = -1;
    a_src[i] = tok >= 0 ? x + (size_t)tok * hidden + l_chunk[i] * 8 : nullptr;
    b_src[i] = wt + (size_t)l_row[i] * hidden + l_chunk[i] * 8;
  }
  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = a_src[i] ? *reinterpret_cast<const u32x4*>(a_src[i] + k0) : u32x4{0, 0, 0, 0};
      rb[i] = *reinterpret_cast<const u32x4*>(b_src[i] + k0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&sm.ab.a[buf][l_row[i]][l_chunk[i] * 8]) = ra[i];
      *reinterpret_cast<u32x4*>(&sm.ab.b[buf][l_row[i]][l_chunk[i] * 8]) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int n_k = hidden / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  for (int kt = 0; kt < n_k; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_k) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&sm.ab.a[buf][wm * 64 + i * 32 + lr][ks * 16 + lk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&sm.ab.b[buf][wn * 64 + j * 32 + lr][ks * 16 + lk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < n_k) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: fp32 tile -> LDS ------------------------------------------
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int c = wn * 64 + j * 32 + (lane & 31);
        sm.c[r][c] = acc[i][j][v];
      }
  __syncthreads();

  if (head < hq + hkv) {
    // Q or K head: rotate-half pairs (e, e+64), 8 pairs per unit.
    const bool is_q = head < hq;
    const int g = head - hq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + 256 * i;
      const int m = u >> 3, c = u & 7;
      const int r = sm.row_req[m];
      if (r < 0) continue;
      const int idx = sm.row_idx[m];
      uint16_t* dst;
      if (is_q) {
        if (!q_out) continue;
        dst = q_out + ((size_t)(m0 + m) * hq + head) * 128;
      } else {
        const int page = page_of(lay, n_pages, r, idx);
        if (page < 0) continue;
        dst = kpool + (((size_t)page * hkv + g) * kPage + (idx & (kPage - 1))) * 128;
      }
      const float* tab = lay.rope_tab + (size_t)rope_pos(lay, r, idx) * 128 + c * 16;
      float olo[8], ohi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float lo = sm.c[m][c * 8 + e], hi = sm.c[m][64 + c * 8 + e];
        const float cs = tab[2 * e], sn = tab[2 * e + 1];
        olo[e] = lo * cs - hi * sn;
        ohi[e] = lo * sn + hi * cs;
      }
      u32x4 plo, phi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        plo[e] = pack_bf2(olo[2 * e], olo[2 * e + 1]);
        phi[e] = pack_bf2(ohi[2 * e], ohi[2 * e + 1]);
      }
      *reinterpret_cast<u32x4*>(dst + c * 8) = plo;
      *reinterpret_cast<u32x4*>(dst + 64 + c * 8) = phi;
    }
  } else {
    // V head: page layout [d][slot]; consecutive lanes take consecutive rows.
    const int g = head - hq - hkv;
    for (int u = tid; u < BM * 128; u += 256) {
      const int m = u & (BM - 1), e = u >> 7;
      const int r = sm.row_req[m];
      if (r < 0) continue;
      const int idx = sm.row_idx[m];
      const int page = page_of(lay, n_pages, r, idx);
      if (page < 0) continue;
      vpool[(((size_t)page * hkv + g) * 128 + e) * kPage + (idx & (kPage - 1))] = f2bf(sm.c[m][e]);
    }
  }
}

// fp32 storage: one workgroup per (row, head), one lane per rotate-half pair
// (or per element for V); dot products accumulate in index order.
template <int D>
__global__ __launch_bounds__(128) void qkv_rows_f32(
    const float* __restrict__ x, int hidden, const int32_t* __restrict__ rows, int n_rows,
    const float* __restrict__ w, int head0, sx_layout lay, int n_pages, float* __restrict__ kpool,
    float* __restrict__ vpool, float* __restrict__ q_out, int hq, int hkv) {
  extern __shared__ float xs[];
  const int m = blockIdx.x;
  const int head = head0 + blockIdx.y;
  const int tok = rows[m];
  const int r = find_request(lay.seq_start, lay.n_req, tok);
  if (r < 0) return;
  const int idx = tok - lay.seq_start[r];
  for (int c = threadIdx.x; c < hidden; c += blockDim.x) xs[c] = x[(size_t)tok * hidden + c];
  __syncthreads();
  const float* wt = w + (size_t)head * D * hidden;
  if (head < hq + hkv) {
    const int e = threadIdx.x;
    if (e >= D / 2) return;
    float lo = 0.f, hi = 0.f;
    for (int c = 0; c < hidden; ++c) {
      lo = fmaf(xs[c], wt[(size_t)e * hidden + c], lo);
      hi = fmaf(xs[c], wt[(size_t)(e + D / 2) * hidden + c], hi);
    }
    const float* tab = lay.rope_tab + (size_t)rope_pos(lay, r, idx) * D + 2 * e;
    const float olo = lo * tab[0] - hi * tab[1];
    const float ohi = lo * tab[1] + hi * tab[0];
    float* dst;
    if (head < hq) {
      if (!q_out) return;
      dst = q_out + ((size_t)m * hq + head) * D;
    } else {
      const int page = page_of(lay, n_pages, r, idx);
      if (page < 0) return;
      dst = kpool + (((size_t)page * hkv + (head - hq)) * kPage + (idx & (kPage - 1))) * D;
    }
    dst[e] = olo;
    dst[e + D / 2] = ohi;
  } else {
    const int page = page_of(lay, n_pages, r, idx);
    if (page < 0) return;
    const int g = head - hq - hkv;
    for (int e = threadIdx.x; e < D; e += blockDim.x) {
      float s = 0.f;
      for (int c = 0; c < hidden; ++c) s = fmaf(xs[c], wt[(size_t)e * hidden + c], s);
      vpool[(((size_t)page * hkv + g) * D + e) * kPage + (idx & (kPage - 1))] = s;
    }
  }
}

}  // namespace

sx_status launch_recompute(const sx_dims& dims, const sx_layout& lay, const void* x,
                           const int32_t* rows, int n_rows, const void* w_qkv,
                           const sx_pages& kv, void* q_out, hipStream_t stream) {
  if (n_rows == 0) return SX_OK;
  const int hq = dims.n_q_heads, hkv = dims.n_kv_heads;
  const int head0 = q_out ? 0 : hq;
  const int n_heads = hq + 2 * hkv - head0;
  if (dims.dtype == SX_BF16) {
    const int mt = (n_rows + BM - 1) / BM;
    const int total = mt * n_heads;
    const int grid = ((total + 7) / 8) * 8;
    const size_t smem = sizeof(GemmSmem);
    const sx_status st = allow_lds((const void*)qkv_gemm_bf16, smem, "sx_recompute_kv");
    if (st != SX_OK) return st;
    qkv_gemm_bf16<<<grid, 256, smem, stream>>>(
        (const uint16_t*)x, dims.hidden, rows, n_rows, (const uint16_t*)w_qkv, head0, mt, n_heads,
        lay, kv.n_pages, (uint16_t*)kv.k, (uint16_t*)kv.v, (uint16_t*)q_out, hq, hkv);
  } else {
    dim3 grid(n_rows, n_heads);
    const size_t smem = (size_t)dims.hidden * sizeof(float);
    if (dims.head_dim == 64)
      qkv_rows_f32<64><<<grid, 128, smem, stream>>>((const float*)x, dims.hidden, rows, n_rows,
                                                    (const float*)w_qkv, head0, lay, kv.n_pages,
                                                    (float*)kv.k, (float*)kv.v, (float*)q_out, hq, hkv);
    else
      qkv_rows_f32<128><<<grid, 128, smem, stream>>>((const float*)x, dims.hidden, rows, n_rows,
                                                     (const float*)w_qkv, head0, lay, kv.n_pages,
                                                     (float*)kv.k, (float*)kv.v, (float*)q_out, hq, hkv);
  }
  return check_launch("sx_recompute_kv");
}

}  // namespace sx
