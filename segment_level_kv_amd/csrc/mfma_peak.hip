// Measured MFMA throughput of the device: the reference the sparse-attention
// utilisation is also quoted against, besides the data-sheet peak.  Every
// wave issues back-to-back v_mfma_f32_32x32x16_bf16 (the instruction the
// attention and projection kernels use), eight in a row on one accumulator
// and then eight on another (gfx950 issues a dependent chain on one
// accumulator faster than MFMAs alternating between accumulators), eight
// waves per workgroup (two per SIMD at one workgroup per compute unit).
// Operands are either small constants or random bf16 values in [-2, 2)
// taken from eight register sets in turn, like the K, V and probability
// fragments of the attention: with random operands the chip draws more power
// and holds a lower clock, so the two rates bracket what MFMA-bound kernels
// can reach on real data.  Each wave stores one reduced value so nothing is
// optimised away.
#include "sx_device.hpp"
#include "sx_internal.hpp"

namespace sx {

namespace {

constexpr int kProbeThreads = 512;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {   // integer hash (operand values only)
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <bool RANDOM>
__global__ __launch_bounds__(kProbeThreads) void mfma_peak_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float va, vb;
      if (RANDOM) {
        const uint32_t h = mix32((blockIdx.x * kProbeThreads + threadIdx.x) * 64u + r * 8u + i);
        va = (float)(h & 0xffffu) * (1.f / 16384.f) - 2.f;
        vb = (float)(h >> 16) * (1.f / 16384.f) - 2.f;
      } else {
        va = 0.001f * (float)((lane + i) & 7);
        vb = 0.002f * (float)((lane * 3 + i) & 7);
      }
      a[r][i] = (__bf16)va;
      b[r][i] = (__bf16)vb;
    }
  f32x16 c0 = f32x16{}, c1 = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r], b[r], c0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 8; ++r) c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(r + 3) & 7], b[(r + 5) & 7], c1, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v];
  if (lane == 0) out[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = s;
}

}  // namespace

sx_status launch_mfma_peak(int n_workgroups, int iters, int random_operands, float* out, hipStream_t stream) {
  if (random_operands)
    mfma_peak_kernel<true><<<n_workgroups, kProbeThreads, 0, stream>>>(out, iters);
  else
    mfma_peak_kernel<false><<<n_workgroups, kProbeThreads, 0, stream>>>(out, iters);
  return check_launch("sx_mfma_peak_probe");
}

}  // namespace sx
