// Fused copy-Delta-RoPE of reused KV pages (SparseX paper §3.1, delta
// equation: k_{p'+j} <- R_{p'-p} k_{p+j}, v_{p'+j} <- v_{p+j}; §4.4 copy
// semantics; §4.5 the worker's fused kernel).
//
// HBM-bound: every byte is read once and written once.  One workgroup per
// page-granular job; 16-byte loads/stores, consecutive lanes on consecutive
// 16-byte chunks of a page, so a full-page job streams each 4 KB (bf16,
// d=128) K page-head and V page-head with fully coalesced accesses.  A lane
// owns element chunk c of the first half of a key row and the matching
// chunk of the second half, so the rotate-half pairs (e, e+d/2) meet in one
// lane with no exchange.
#include "sx_device.hpp"
#include "sx_internal.hpp"

namespace sx {

template <typename S> struct Vec16;
template <> struct Vec16<uint16_t> { static constexpr int N = 8; };
template <> struct Vec16<float> { static constexpr int N = 4; };

__device__ __forceinline__ void unpack16(const u32x4& v, float* f, uint16_t*) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(const u32x4& v, float* f, float*) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}
__device__ __forceinline__ u32x4 pack16(const float* f, uint16_t*) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf2(f[2 * i], f[2 * i + 1]);
  return v;
}
__device__ __forceinline__ u32x4 pack16(const float* f, float*) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
  return v;
}

template <typename S, int D>
__global__ __launch_bounds__(256) void realign_kernel(
    const S* __restrict__ ksrc, const S* __restrict__ vsrc, S* __restrict__ kdst,
    S* __restrict__ vdst, int n_src_pages, int n_dst_pages, int hkv,
    const sx_realign_job* __restrict__ jobs, const float* __restrict__ rope_tab, int rope_len) {
  constexpr int N = Vec16<S>::N;           // elements per 16-byte chunk
  constexpr int UPR = (D / 2) / N;         // chunk pairs per key row
  constexpr int VPC = kPage / N;           // 16-byte chunks per V page row (one d)
  const sx_realign_job jb = jobs[blockIdx.x];
  const int n = jb.n_tok;
  if (jb.src_page < 0 || jb.src_page >= n_src_pages || jb.dst_page < 0 ||
      jb.dst_page >= n_dst_pages || n <= 0 || jb.src_slot < 0 || jb.dst_slot < 0 ||
      jb.src_slot + n > kPage || jb.dst_slot + n > kPage)
    return;
  const int ad = jb.delta < 0 ? -jb.delta : jb.delta;
  if (ad >= rope_len) return;
  const float sgn = jb.delta < 0 ? -1.f : 1.f;
  const size_t head_elems = (size_t)kPage * D;
  const S* ks = ksrc + (size_t)jb.src_page * hkv * head_elems;
  S* kd = kdst + (size_t)jb.dst_page * hkv * head_elems;
  const float* tab = rope_tab + (size_t)ad * D;   // [D/2][2] cos, sin

  // ---- keys: rotate by R_delta -------------------------------------------
  const int k_units = hkv * n * UPR;
  for (int u = threadIdx.x; u < k_units; u += blockDim.x) {
    const int c = u % UPR;
    const int t = (u / UPR) % n;
    const int h = u / (UPR * n);
    const S* src = ks + h * head_elems + (size_t)(jb.src_slot + t) * D + c * N;
    S* dst = kd + h * head_elems + (size_t)(jb.dst_slot + t) * D + c * N;
    const u32x4 lo_raw = *reinterpret_cast<const u32x4*>(src);
    const u32x4 hi_raw = *reinterpret_cast<const u32x4*>(src + D / 2);
    float lo[N], hi[N], olo[N], ohi[N];
    unpack16(lo_raw, lo, (S*)nullptr);
    unpack16(hi_raw, hi, (S*)nullptr);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = c * N + i;
      const float cs = tab[2 * e];
      const float sn = sgn * tab[2 * e + 1];
      olo[i] = lo[i] * cs - hi[i] * sn;
      ohi[i] = lo[i] * sn + hi[i] * cs;
    }
    *reinterpret_cast<u32x4*>(dst) = pack16(olo, (S*)nullptr);
    *reinterpret_cast<u32x4*>(dst + D / 2) = pack16(ohi, (S*)nullptr);
  }

  // ---- values: plain copy of the page columns ------------------------------
  const S* vs = vsrc + (size_t)jb.src_page * hkv * head_elems;
  S* vd = vdst + (size_t)jb.dst_page * hkv * head_elems;
  if (n == kPage && jb.src_slot == 0 && jb.dst_slot == 0) {
    const int v_units = hkv * D * VPC;        // whole pages, 16 B at a time
    for (int u = threadIdx.x; u < v_units; u += blockDim.x) {
      reinterpret_cast<u32x4*>(vd)[u] = reinterpret_cast<const u32x4*>(vs)[u];
    }
  } else {
    const int v_elems = hkv * D * n;
    for (int u = threadIdx.x; u < v_elems; u += blockDim.x) {
      const int t = u % n;
      const int row = u / n;                  // h * D + d
      vd[(size_t)row * kPage + jb.dst_slot + t] = vs[(size_t)row * kPage + jb.src_slot + t];
    }
  }
}

sx_status launch_realign(const sx_dims& dims, const sx_layout& lay, const sx_pages& src,
                         const sx_pages& dst, const sx_realign_job* jobs, int n_jobs,
                         hipStream_t stream) {
  if (n_jobs == 0) return SX_OK;
  dim3 grid(n_jobs), block(256);
  if (dims.dtype == SX_BF16) {
    realign_kernel<uint16_t, 128><<<grid, block, 0, stream>>>(
        (const uint16_t*)src.k, (const uint16_t*)src.v, (uint16_t*)dst.k, (uint16_t*)dst.v,
        src.n_pages, dst.n_pages, dims.n_kv_heads, jobs, lay.rope_tab, lay.rope_len);
  } else if (dims.head_dim == 64) {
    realign_kernel<float, 64><<<grid, block, 0, stream>>>(
        (const float*)src.k, (const float*)src.v, (float*)dst.k, (float*)dst.v, src.n_pages,
        dst.n_pages, dims.n_kv_heads, jobs, lay.rope_tab, lay.rope_len);
  } else {
    realign_kernel<float, 128><<<grid, block, 0, stream>>>(
        (const float*)src.k, (const float*)src.v, (float*)dst.k, (float*)dst.v, src.n_pages,
        dst.n_pages, dims.n_kv_heads, jobs, lay.rope_tab, lay.rope_len);
  }
  return check_launch("sx_rope_realign");
}

}  // namespace sx
