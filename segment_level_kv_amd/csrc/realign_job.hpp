// One page-granular job of the fused copy-Delta-RoPE (SparseX paper §3.1,
// delta equation: k_{p'+j} <- R_{p'-p} k_{p+j}, v_{p'+j} <- v_{p+j}; §4.4
// copy semantics), done by the nthreads threads tid = 0..nthreads-1 of a
// workgroup.  Shared by the realign kernel (one job per workgroup) and the
// projection kernel's realign workers (a strided list of jobs each).
//
// 16-byte loads/stores, consecutive threads on consecutive 16-byte chunks
// of a page, so a full-page job streams each 4 KB (bf16, d=128) K page-head
// and V page-head with fully coalesced accesses.  A thread owns element
// chunk c of the first half of a key row and the matching chunk of the
// second half, so the rotate-half pairs (e, e+d/2) meet in one thread with no
// exchange.  A job with a page, slot or count out of range, or |delta| not
// below rope_len, is skipped.
#pragma once

#include "sx_device.hpp"

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

// The rotation of one pair (lo, hi) = (x_e, x_{e+d/2}) by (cos, sin), with
// the rounding fixed (one product, then one fused multiply-add), so every
// code path that rotates gives the same bits.
__device__ __forceinline__ float rot_lo(float lo, float hi, float cs, float sn) {
  return fmaf(lo, cs, -(hi * sn));
}
__device__ __forceinline__ float rot_hi(float lo, float hi, float cs, float sn) {
  return fmaf(lo, sn, hi * cs);
}

template <typename S, int D>
__device__ __forceinline__ void realign_one_job(
    const sx_realign_job& jb, const S* __restrict__ ksrc, const S* __restrict__ vsrc,
    S* __restrict__ kdst, S* __restrict__ vdst, int n_src_pages, int n_dst_pages, int hkv,
    const float* __restrict__ rope_tab, int rope_len, int tid, int nthreads) {
  constexpr int N = Vec16<S>::N;           // elements per 16-byte chunk
  constexpr int UPR = (D / 2) / N;         // chunk pairs per key row
  constexpr int VPC = kPage / N;           // 16-byte chunks per V page row (one d)
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
  for (int u = tid; u < k_units; u += nthreads) {
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
      olo[i] = rot_lo(lo[i], hi[i], cs, sn);
      ohi[i] = rot_hi(lo[i], hi[i], cs, sn);
    }
    *reinterpret_cast<u32x4*>(dst) = pack16(olo, (S*)nullptr);
    *reinterpret_cast<u32x4*>(dst + D / 2) = pack16(ohi, (S*)nullptr);
  }

  // ---- values: plain copy of the page columns ------------------------------
  const S* vs = vsrc + (size_t)jb.src_page * hkv * head_elems;
  S* vd = vdst + (size_t)jb.dst_page * hkv * head_elems;
  if (n == kPage && jb.src_slot == 0 && jb.dst_slot == 0) {
    const int v_units = hkv * D * VPC;        // whole pages, 16 B at a time
    for (int u = tid; u < v_units; u += nthreads) {
      reinterpret_cast<u32x4*>(vd)[u] = reinterpret_cast<const u32x4*>(vs)[u];
    }
  } else {
    const int v_elems = hkv * D * n;
    for (int u = tid; u < v_elems; u += nthreads) {
      const int t = u % n;
      const int row = u / n;                  // h * D + d
      vd[(size_t)row * kPage + jb.dst_slot + t] = vs[(size_t)row * kPage + jb.src_slot + t];
    }
  }
}

// A run of jobs done by one workgroup of nthreads (a multiple of 64) threads,
// RB jobs at a time: when all RB are whole-page bf16 jobs every load of the
// RB pages is issued before the first store, so a single workgroup keeps
// enough bytes in flight to stream at a useful rate; any other group of
// jobs goes through realign_one_job one by one.  Same results as
// realign_one_job on each job.
template <int RB, int NT>
__device__ __forceinline__ void realign_job_run(
    const sx_realign_job* __restrict__ jobs, int j0, int j1, const uint16_t* __restrict__ ksrc,
    const uint16_t* __restrict__ vsrc, uint16_t* __restrict__ kdst, uint16_t* __restrict__ vdst,
    int n_src_pages, int n_dst_pages, int hkv, const float* __restrict__ rope_tab, int rope_len,
    int tid) {
  constexpr int D = 128, N = 8, UPR = (D / 2) / N;     // 8 chunk pairs per key row
  constexpr int HE = kPage * D;                         // elements per page-head
  for (int j = j0; j < j1; j += RB) {
    sx_realign_job jb[RB];
    bool fast = j + RB <= j1 && hkv * kPage * UPR == 2 * NT && hkv * D * 2 == 4 * NT;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      jb[i] = jobs[min(j + i, j1 - 1)];
      const int ad = jb[i].delta < 0 ? -jb[i].delta : jb[i].delta;
      fast = fast && jb[i].n_tok == kPage && jb[i].src_slot == 0 && jb[i].dst_slot == 0 &&
             jb[i].src_page >= 0 && jb[i].src_page < n_src_pages && jb[i].dst_page >= 0 &&
             jb[i].dst_page < n_dst_pages && ad < rope_len;
    }
    if (!fast) {
      for (int i = j; i < min(j + RB, j1); ++i)
        realign_one_job<uint16_t, D>(jobs[i], ksrc, vsrc, kdst, vdst, n_src_pages, n_dst_pages, hkv,
                                     rope_tab, rope_len, tid, NT);
      continue;
    }
    // whole pages: key unit u = tid + NT r (r < 2) is (head, token, chunk pair
    // c = tid % 8); value chunk u = tid + NT r (r < 4) of the page's V block
    const int c = tid % UPR;
    u32x4 klo[RB][2], khi[RB][2], vv[RB][4];
    f32x4 tb[RB][4];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const uint16_t* ks = ksrc + (size_t)jb[i].src_page * hkv * HE;
      const uint16_t* vs = vsrc + (size_t)jb[i].src_page * hkv * HE;
      const int ad = jb[i].delta < 0 ? -jb[i].delta : jb[i].delta;
      const f32x4* tab = reinterpret_cast<const f32x4*>(rope_tab + (size_t)ad * D + c * N * 2);
#pragma unroll
      for (int q = 0; q < 4; ++q) tb[i][q] = tab[q];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int u = tid + NT * r;
        const uint16_t* src = ks + (size_t)(u / UPR) * D + c * N;     // (head, token) rows are contiguous
        klo[i][r] = *reinterpret_cast<const u32x4*>(src);
        khi[i][r] = *reinterpret_cast<const u32x4*>(src + D / 2);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) vv[i][r] = reinterpret_cast<const u32x4*>(vs)[tid + NT * r];
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      uint16_t* kd = kdst + (size_t)jb[i].dst_page * hkv * HE;
      uint16_t* vd = vdst + (size_t)jb[i].dst_page * hkv * HE;
      const float sgn = jb[i].delta < 0 ? -1.f : 1.f;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int u = tid + NT * r;
        float lo[N], hi[N], olo[N], ohi[N];
        unpack16(klo[i][r], lo, (uint16_t*)nullptr);
        unpack16(khi[i][r], hi, (uint16_t*)nullptr);
#pragma unroll
        for (int e = 0; e < N; ++e) {
          const float cs = tb[i][e >> 1][2 * (e & 1)];
          const float sn = sgn * tb[i][e >> 1][2 * (e & 1) + 1];
          olo[e] = rot_lo(lo[e], hi[e], cs, sn);
          ohi[e] = rot_hi(lo[e], hi[e], cs, sn);
        }
        uint16_t* dst = kd + (size_t)(u / UPR) * D + c * N;
        *reinterpret_cast<u32x4*>(dst) = pack16(olo, (uint16_t*)nullptr);
        *reinterpret_cast<u32x4*>(dst + D / 2) = pack16(ohi, (uint16_t*)nullptr);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) reinterpret_cast<u32x4*>(vd)[tid + NT * r] = vv[i][r];
    }
  }
}

}  // namespace sx
