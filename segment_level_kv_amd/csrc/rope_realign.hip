// Fused copy-Delta-RoPE of reused KV pages (SparseX paper §3.1, delta
// equation: k_{p'+j} <- R_{p'-p} k_{p+j}, v_{p'+j} <- v_{p+j}; §4.4 copy
// semantics; §4.5 the worker's fused kernel).
//
// HBM-bound: every byte is read once and written once.  One workgroup per
// page-granular job (the job body is in realign_job.hpp).
#include "realign_job.hpp"
#include "sx_device.hpp"
#include "sx_internal.hpp"

namespace sx {

template <typename S, int D>
__global__ __launch_bounds__(256) void realign_kernel(
    const S* __restrict__ ksrc, const S* __restrict__ vsrc, S* __restrict__ kdst,
    S* __restrict__ vdst, int n_src_pages, int n_dst_pages, int hkv,
    const sx_realign_job* __restrict__ jobs, const float* __restrict__ rope_tab, int rope_len) {
  realign_one_job<S, D>(jobs[blockIdx.x], ksrc, vsrc, kdst, vdst, n_src_pages, n_dst_pages, hkv,
                        rope_tab, rope_len, threadIdx.x, blockDim.x);
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
