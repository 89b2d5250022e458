// Device-side helpers shared by the libsx kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sx.h"

namespace sx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPage = 16;      // tokens per KV page
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 <-> fp32.  bf16 storage is handled as raw 16-bit patterns.
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// Two floats -> two bf16 (RNE) in one 32-bit word, lo in bits 0-15
// (a single v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

// Two fp32 values -> packed fp16 pair (round to nearest even), and back.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
}
__device__ __forceinline__ f32x2_t unpack_h2(uint32_t v) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2_t, v), f32x2_t);
}

// One 16-byte chunk per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane L writes bytes [16 L, 16 L + 16) after
// the wave's LDS base `lds` (wave-uniform, passed in M0).  It is issued as
// inline asm rather than through the compiler builtin: the compiler counts
// the builtin as a FLAT access that may write LDS, and while one is
// pending its wait-count pass can only wait for an LDS read with
// lgkmcnt(0), which drains every LDS read in flight before the first
// operand is used.  The asm has no register result.  The compiler does not
// count these loads; since loads complete in issue order, that only makes
// its own vmcnt waits stricter.  Callers order the LDS writes themselves,
// with vmcnt waits and barriers before any wave reads the bytes.
__device__ __forceinline__ void copy16_to_lds(const void* gsrc, const void* lds) {
  typedef __attribute__((address_space(3))) const void* lds_ptr_t;
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(m0) : "memory");
}

// Request owning packed token `tok` (seq_start ascending, n_req+1 entries).
// Returns -1 if tok is outside [seq_start[0], seq_start[n_req]).
__device__ __forceinline__ int find_request(const int32_t* __restrict__ seq_start, int n_req, int tok) {
  if (tok < seq_start[0] || tok >= seq_start[n_req]) return -1;
  int lo = 0, hi = n_req - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (seq_start[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Physical page of token index i of request r, or -1 if any index is out of
// range (the kernels then skip the access).
__device__ __forceinline__ int page_of(const sx_layout& L, int n_pages, int r, int i) {
  int pi = i / kPage;
  if (i < 0 || pi >= L.max_pages) return -1;
  int p = L.block_table[(size_t)r * L.max_pages + pi];
  return (p >= 0 && p < n_pages) ? p : -1;
}

__device__ __forceinline__ int rope_pos(const sx_layout& L, int r, int i) {
  int m = i + (L.pos_offset ? L.pos_offset[r] : 0);
  // Out-of-table positions are clamped (wrong values, never a stray read).
  return m < 0 ? 0 : (m >= L.rope_len ? L.rope_len - 1 : m);
}

}  // namespace sx
