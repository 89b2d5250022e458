// Measured MFMA throughput of the device: the reference the sparse-attention
// utilisation is quoted against besides the data-sheet peak.  Every wave
// issues back-to-back v_mfma_f32_32x32x16_bf16 (the instruction the
// attention and projection kernels use) on four independent accumulators,
// eight waves per workgroup (two per SIMD), several workgroups per compute
// unit.  Each wave stores one reduced value so nothing is optimised away.
#include "sx_device.hpp"
#include "sx_internal.hpp"

namespace sx {

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeMfmaPerIter = 16;

__global__ __launch_bounds__(kProbeThreads) void mfma_peak_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((lane + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((lane * 3 + i) & 7));
  }
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < kProbeMfmaPerIter / 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[i][v];
  if (lane == 0) out[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = s;
}

}  // namespace

sx_status launch_mfma_peak(int n_workgroups, int iters, float* out, hipStream_t stream) {
  mfma_peak_kernel<<<n_workgroups, kProbeThreads, 0, stream>>>(out, iters);
  return check_launch("sx_mfma_peak_probe");
}

}  // namespace sx
