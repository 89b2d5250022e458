// Decode attention over the mixed paged cache ("SparseX: Efficient
// Segment-Level KV Cache Sharing for Interleaved LLM Serving", §4.5 last
// paragraph: after the first prefill pass, decode reads the realigned and
// recomputed blocks through the block table).  For each request r with
// T_r tokens in its cache (the new token's K/V already written) and query
// head h of kv group g:
//   o[r][h] = sum_{j < T_r} softmax_j(q[r][h] . k_j^g / sqrt(d)) v_j^g.
//
// One query row per request makes this an HBM stream: every key and value of
// the request is read once per kv head, against 2*G flops per byte pair.
// Design (gfx950):
//   - workgroups (slot s, kv head g, request r), 4 waves; a "unit" is 32 keys
//     = two 16-slot pages.  Wave w of slot s takes units s + S*(w + 4i), so
//     one request's keys are spread over S*4 waves that all run at once;
//   - Q K^T per page with v_mfma_f32_16x16x32_bf16: A = the page's 16 keys
//     (row = lane%16, straight from the [slot][d] page), B = Q^T with the G
//     query heads of the group as columns (the other 16-G columns are zero);
//     D row 4*(lane/16)+v is key slot 4*(lane/16)+v, column lane%16 the head;
//   - P V with the same instruction, A = V^T (row = d, from the transposed
//     [d][slot] page), B = P^T.  The contraction index k = 8*(lane/16)+i is
//     mapped to key slot 4*(lane/16)+i of the first page for i < 4 and of the
//     second page for i >= 4: exactly the scores the lane already holds from
//     Q K^T, so P needs no data movement, and V^T is two 8-byte loads;
//   - online softmax in the log2 domain per wave; the 4 waves are merged in
//     LDS; one fp32 partial (m, l, o) per (request, head, slot) goes to the
//     workspace and decode_merge combines the slots in a fixed order.
#include <mutex>

#include "sx_device.hpp"
#include "sx_internal.hpp"

namespace sx {
namespace {

// Scratch of sx_decode_attn_noalloc: the partial results of decode_fwd live
// in this file-scope array instead of a caller workspace.  Every GPU the
// library runs on holds its own copy until the process ends.  In host code
// the name `scratch` is only a stand-in; the device address of this GPU's
// copy comes from hipGetSymbolAddress (decode_scratch below) and is the only
// thing passed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kUnitKeys = 32;
constexpr int kDecD = 128;                 // head_dim of the bf16 path
constexpr int kPartStride = kDecD + 2;     // o[128], m, l per (request, head, slot)
constexpr int kTargetWG = 512;             // two workgroups per CU

__device__ __forceinline__ float wave_max16(float x) {
  // max over the lanes sharing lane % 16 (lanes l, l^16, l^32, l^48)
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum16(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

struct DecSmem {
  float m[kDecWaves][16];
  float l[kDecWaves][16];
  float o[kDecWaves][kDecD][16];
};

// One unit's operands in registers: K of both pages (A operand of Q K^T),
// V^T of both pages (A operand of P V) and how many keys each page holds.
struct DecUnit {
  bf16x8 kA[4], kB[4];
  u32x2 vA[8], vB[8];
  int na, nb;
};

// Every page is read through a buffer resource built in scalar registers from
// its wave-uniform base (one kv head's 4 KB of K or V), with a fixed 32-bit
// per-lane offset: no per-unit vector address arithmetic, and the hardware
// range check returns zeros for any offset outside the 4 KB.
constexpr uint32_t kBufWord3 = 0x00020000;   // raw buffer, 32-bit data format
constexpr int kHeadPageBytes = kPage * kDecD * 2;

// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ uint64_t uniform64(uint64_t a) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(uint64_t base) {
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char*>(uniform64(base)), (short)0,
                                           kHeadPageBytes, kBufWord3);
}

__device__ __forceinline__ void load_unit(DecUnit& U, int u, int T, const int32_t* __restrict__ btr,
                                          int max_pages, int n_pages, uint64_t kg, uint64_t vg,
                                          uint64_t page_bytes, uint32_t k_lane, uint32_t v_lane) {
  // keys of the unit held by each page, and the pages (bounds-checked)
  const int key0 = u * kUnitKeys;
  int na = min(T - key0, kPage);
  int nb = min(max(T - key0 - kPage, 0), kPage);
  const int pia = 2 * u, pib = 2 * u + 1;
  int ida = pia < max_pages ? btr[pia] : -1;
  int idb = (nb > 0 && pib < max_pages) ? btr[pib] : -1;
  if ((unsigned)ida >= (unsigned)n_pages) { ida = 0; na = 0; }
  if ((unsigned)idb >= (unsigned)n_pages) { idb = ida; nb = 0; }
  U.na = na;
  U.nb = nb;
  const __amdgpu_buffer_rsrc_t ka = page_rsrc(kg + (uint64_t)ida * page_bytes);
  const __amdgpu_buffer_rsrc_t kb = page_rsrc(kg + (uint64_t)idb * page_bytes);
  const __amdgpu_buffer_rsrc_t va = page_rsrc(vg + (uint64_t)ida * page_bytes);
  const __amdgpu_buffer_rsrc_t vb = page_rsrc(vg + (uint64_t)idb * page_bytes);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    U.kA[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ka, k_lane + ks * 64, 0, 0));
    U.kB[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kb, k_lane + ks * 64, 0, 0));
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    U.vA[b] = __builtin_amdgcn_raw_buffer_load_b64(va, v_lane + b * 512, 0, 0);
    U.vB[b] = __builtin_amdgcn_raw_buffer_load_b64(vb, v_lane + b * 512, 0, 0);
  }
}

// Online-softmax step of one unit for the lane's head (column lane % 16).
__device__ __forceinline__ void unit_math(DecUnit& U, const bf16x8 (&qf)[4], float scale_log2, int grp,
                                          float& m, float& lsum, f32x4 (&o)[8]) {
  // S^T = K Q^T for both pages
  f32x4 sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    sA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(U.kA[ks], qf[ks], sA, 0, 0, 0);
    sB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(U.kB[ks], qf[ks], sB, 0, 0, 0);
  }
  float x[8];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    x[v] = sA[v] * scale_log2;
    x[4 + v] = sB[v] * scale_log2;
  }
  const int na = U.na, nb = U.nb;
  if (na < kPage || nb < kPage) {   // ragged last unit or a bad page id: mask keys, zero their v
    uint32_t keep_a[2], keep_b[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int sl = 4 * grp + 2 * h;
      keep_a[h] = (sl < na ? 0xffffu : 0u) | (sl + 1 < na ? 0xffff0000u : 0u);
      keep_b[h] = (sl < nb ? 0xffffu : 0u) | (sl + 1 < nb ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (4 * grp + v >= na) x[v] = -INFINITY;
      if (4 * grp + v >= nb) x[4 + v] = -INFINITY;
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      U.vA[b][0] &= keep_a[0]; U.vA[b][1] &= keep_a[1];
      U.vB[b][0] &= keep_b[0]; U.vB[b][1] &= keep_b[1];
    }
  }
  float mx = x[0];
#pragma unroll
  for (int v = 1; v < 8; ++v) mx = fmaxf(mx, x[v]);
  mx = wave_max16(mx);
  const float m_new = fmaxf(m, mx);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m - m_use);
  float p[8], ps = 0.f;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    p[v] = __builtin_amdgcn_exp2f(x[v] - m_use);
    ps += p[v];
  }
  lsum = lsum * alpha + ps;
  m = m_new;
  const uint32_t w0 = pack_bf2(p[0], p[1]), w1 = pack_bf2(p[2], p[3]);
  const uint32_t w2 = pack_bf2(p[4], p[5]), w3 = pack_bf2(p[6], p[7]);
  const bf16x8 P = __builtin_bit_cast(bf16x8, u32x4{w0, w1, w2, w3});
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    o[b] *= alpha;
    const bf16x8 vt = __builtin_bit_cast(bf16x8, u32x4{U.vA[b][0], U.vA[b][1], U.vB[b][0], U.vB[b][1]});
    o[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, P, o[b], 0, 0, 0);
  }
}

__global__ __launch_bounds__(kDecThreads, 2) void decode_fwd(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kpool,
    const uint16_t* __restrict__ vpool, int n_pages, const int32_t* __restrict__ seq_start,
    const int32_t* __restrict__ block_table, int max_pages, int hq, int hkv, int n_slots,
    float scale_log2, float* __restrict__ part) {
  __shared__ DecSmem sm;
  const int s = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int G = hq / hkv;
  const int lane = threadIdx.x & 63;
  // wave index as a scalar: unit indices and page ids are wave-uniform, so
  // the block-table reads become scalar loads that do not wait on the
  // vector loads of the unit in flight
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int T = seq_start[r + 1] - seq_start[r];
  const int n_u = T > 0 ? (T + kUnitKeys - 1) / kUnitKeys : 0;

  // Q^T fragments: head g*G + col, dims ks*32 + 8*grp + i
  bf16x8 qf[4];
  if (col < G) {
    const uint16_t* qp = q + ((size_t)r * hq + (size_t)g * G + col) * kDecD + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
  } else {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = bf16x8{};
  }

  const uint64_t page_bytes = (uint64_t)hkv * kPage * kDecD * 2;
  const uint64_t kg = uniform64(reinterpret_cast<uint64_t>(kpool) + (uint64_t)g * kHeadPageBytes);
  const uint64_t vg = uniform64(reinterpret_cast<uint64_t>(vpool) + (uint64_t)g * kHeadPageBytes);
  // K page [slot][d]: lane reads slot col, dims 8*grp + 32*ks (16 bytes);
  // V page [d][slot]: lane reads d = col + 16*b, slots 4*grp..4*grp+3 (8 bytes)
  const uint32_t k_lane = (uint32_t)(col * kDecD + 8 * grp) * 2;
  const uint32_t v_lane = (uint32_t)(col * kPage + 4 * grp) * 2;
  const int32_t* btr = block_table + (size_t)r * max_pages;

  float m = -INFINITY;     // running max (log2 domain) of head `col`
  float lsum = 0.f;        // this lane's share of the normaliser
  f32x4 o[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Wave w of slot s takes units s + S*w, s + S*(w + 4), ...  One unit's
  // loads are all issued before its math; the other waves of the CU keep
  // the memory pipeline busy meanwhile (a register double buffer, tried,
  // gained nothing: the kernel already streams near the chip's read rate).
  const int stride = n_slots * kDecWaves;
  DecUnit cur;
  for (int u = s + n_slots * w; u < n_u; u += stride) {
    load_unit(cur, u, T, btr, max_pages, n_pages, kg, vg, page_bytes, k_lane, v_lane);
    unit_math(cur, qf, scale_log2, grp, m, lsum, o);
  }

  // merge the 4 waves: lane (col, grp) holds o[d = 16b + 4grp + v][head col]
  lsum = wave_sum16(lsum);
  if (grp == 0) {
    sm.m[w][col] = m;
    sm.l[w][col] = lsum;
  }
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int v = 0; v < 4; ++v) sm.o[w][16 * b + 4 * grp + v][col] = o[b][v];
  __syncthreads();
  float* dst = part + (((size_t)r * hkv + g) * n_slots + s) * (size_t)G * kPartStride;
  for (int e = threadIdx.x; e < G * kDecD; e += kDecThreads) {
    const int j = e / kDecD, d = e % kDecD;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) M = fmaxf(M, sm.m[ww][j]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float acc = 0.f, L = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      const float sc = __builtin_amdgcn_exp2f(sm.m[ww][j] - Mu);
      acc += sc * sm.o[ww][d][j];
      L += sc * sm.l[ww][j];
    }
    dst[(size_t)j * kPartStride + d] = acc;
    if (d == 0) {
      dst[(size_t)j * kPartStride + kDecD] = M;
      dst[(size_t)j * kPartStride + kDecD + 1] = L;
    }
  }
}

// One workgroup of 256 threads per (query head, request): combine the
// slots' partials, normalise, store O (bf16) and the natural-log LSE.
// Slots are taken 64 at a time with one round of loads per chunk: every
// thread loads its element of the chunk's o vectors into registers while
// the chunk's (m, l) pairs go to LDS; the chunks are combined with an
// online rescale, all sums in a fixed order.  A request with no keys gets
// O = 0 and LSE = -inf.
constexpr int kMergeThreads = 256;
constexpr int kMergeChunk = 64;                       // slots per chunk
constexpr int kMergePer = kMergeChunk / (kMergeThreads / kDecD);   // slots per thread per chunk

__global__ __launch_bounds__(kMergeThreads) void decode_merge(const float* __restrict__ part, int hq,
                                                            int hkv, int n_slots,
                                                            uint16_t* __restrict__ o,
                                                            float* __restrict__ lse) {
  __shared__ float cw[kMergeChunk];     // chunk slot weights exp2(m_s - m_run)
  __shared__ float cpar[2];             // rescale of the running sums, chunk normaliser
  __shared__ float half_acc[kDecD];
  const int h = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int G = hq / hkv, g = h / G, j = h % G;
  const size_t slot_stride = (size_t)G * kPartStride;
  const float* src = part + ((size_t)r * hkv + g) * n_slots * slot_stride + (size_t)j * kPartStride;
  const int d = tid & (kDecD - 1), half = tid / kDecD;
  float m_run = -INFINITY;   // wave 0's running max (uniform in wave 0)
  float acc = 0.f, L = 0.f;
  for (int c0 = 0; c0 < n_slots; c0 += kMergeChunk) {
    const int nc = min(kMergeChunk, n_slots - c0);
    float ms = -INFINITY, ls = 0.f;
    if (tid < nc) {
      ms = src[(size_t)(c0 + tid) * slot_stride + kDecD];
      ls = src[(size_t)(c0 + tid) * slot_stride + kDecD + 1];
    }
    float v[kMergePer];
#pragma unroll
    for (int u = 0; u < kMergePer; ++u) {
      const int sl = half + 2 * u;
      v[u] = sl < nc ? src[(size_t)(c0 + sl) * slot_stride + d] : 0.f;
    }
    if (tid < 64) {   // wave 0: chunk max, weights, normaliser
      float cmax = ms;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off));
      const float m_new = fmaxf(m_run, cmax);
      const float mu = m_new == -INFINITY ? 0.f : m_new;
      const float wv = __builtin_amdgcn_exp2f(ms - mu);
      float lc = wv * ls;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) lc += __shfl_xor(lc, off);
      cw[tid] = wv;
      if (tid == 0) {
        cpar[0] = __builtin_amdgcn_exp2f(m_run - mu);
        cpar[1] = lc;
      }
      m_run = m_new;
    }
    __syncthreads();
    const float keep = cpar[0];
    float a = 0.f;
#pragma unroll
    for (int u = 0; u < kMergePer; ++u) a += cw[half + 2 * u] * v[u];   // weight 0 past nc
    acc = acc * keep + a;
    L = L * keep + cpar[1];
    __syncthreads();   // cw/cpar are rewritten by the next chunk
  }
  if (half == 1) half_acc[d] = acc;
  __syncthreads();
  if (half == 0) {
    acc += half_acc[d];
    const float out = L > 0.f ? acc / L : 0.f;
    o[((size_t)r * hq + h) * kDecD + d] = f2bf(out);
    if (lse && tid == 0) lse[(size_t)r * hq + h] = L > 0.f ? (m_run + log2f(L)) * kLn2 : -INFINITY;
  }
}

}  // namespace

int decode_slots(const sx_dims& d, int n_tok, int n_req) {
  const int per = d.n_kv_heads * (n_req > 0 ? n_req : 1);
  int s = (kTargetWG + per - 1) / per;
  const int cap = (n_tok + 4 * kUnitKeys - 1) / (4 * kUnitKeys);   // >= 1 unit per wave
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}

size_t decode_noalloc_capacity() { return kNoAllocScratchBytes; }

// This device's copy of `scratch`, looked up once per device (with that
// device current) and kept.
sx_status decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(SX_EDEVICE, "decode scratch: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(SX_EUNSUPPORTED, "decode scratch: device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(SX_EDEVICE, "decode scratch: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SX_OK;
}

size_t decode_ws_bytes(const sx_dims& d, int n_tok, int n_req) {
  if (d.dtype != SX_BF16) return 0;
  return align256((size_t)n_req * d.n_q_heads * decode_slots(d, n_tok, n_req) * kPartStride *
                  sizeof(float));
}

sx_status launch_decode(const sx_dims& dims, const sx_layout& lay, const void* q, const sx_pages& kv,
                        void* o, float* lse, void* ws, hipStream_t stream) {
  const int hq = dims.n_q_heads, hkv = dims.n_kv_heads;
  const int n_slots = decode_slots(dims, lay.n_tok, lay.n_req);
  float* part = static_cast<float*>(ws);
  const float scale_log2 = kLog2e / sqrtf((float)dims.head_dim);
  decode_fwd<<<dim3(n_slots, hkv, lay.n_req), kDecThreads, 0, stream>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv.k),
      static_cast<const uint16_t*>(kv.v), kv.n_pages, lay.seq_start, lay.block_table, lay.max_pages,
      hq, hkv, n_slots, scale_log2, part);
  sx_status st = check_launch("decode attention");
  if (st != SX_OK) return st;
  decode_merge<<<dim3(hq, lay.n_req), kMergeThreads, 0, stream>>>(part, hq, hkv, n_slots,
                                                                  static_cast<uint16_t*>(o), lse);
  return check_launch("decode merge");
}

}  // namespace sx
