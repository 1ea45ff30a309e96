// Device-side building blocks shared by the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// MFMA wrappers.  Lane layouts (verified on gfx950):
//  16x16xK: A lane l holds row (l % 16), a contiguous K-slice chosen by (l / 16);
//           B lane l holds column (l % 16) with the same K-slice; A and B pair their
//           K elements position by position, so any K permutation applied to both
//           operands gives the same dot products.
//           D lane l holds column (l % 16), rows 4 * (l / 16) + i, i = 0..3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// OCP E4M3 x OCP E4M3, 16x16x128 (format code 0 for both operands, unit scales).
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// two floats to a bf16 pair (round to nearest even), the first in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
}

// ---------------------------------------------------------------------------
// Order-preserving map float -> uint32 (larger float -> larger key); -0 maps to +0 so
// that signed zeros tie.  Key 0 is never produced by a finite or infinite float, so
// "key > 0" admits every candidate.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------------------
// Wave helpers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
// number of set bits of m below this lane
__device__ __forceinline__ uint32_t rank_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}
__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

template <typename T>
__device__ __forceinline__ T uniform(T v) { return __builtin_amdgcn_readfirstlane(v); }

// max / sum over the lanes {l, l^16, l^32, l^48}, with the gfx950 lane swaps (no LDS):
// permlane32_swap(v, v) yields the two 32-lane halves of v side by side, permlane16_swap
// the two 16-lane rows of each half.
__device__ __forceinline__ float wave_max16x4(float v) {
  auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
  auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
}
__device__ __forceinline__ float wave_sum16x4(float v) {
  auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(y[0]) + __uint_as_float(y[1]);
}

// Reduce-scatter of four per-lane partial sums p[0..3] over the four 16-lane groups:
// afterwards lane l holds sum over groups g of p[l / 16] taken at lane (l % 16) + 16 g.
// Uses the gfx950 cross-half (32) and cross-row (16) lane swaps.
__device__ __forceinline__ float reduce_scatter4(float p0, float p1, float p2, float p3) {
  // Step 1: lanes 0-31 keep blocks 0,1 and lanes 32-63 keep blocks 2,3.
  // permlane32_swap(a, b) returns {[a_lo, b_lo], [a_hi, b_hi]} (halves of 32 lanes).
  auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
  auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
  float q0 = __uint_as_float(x[0]) + __uint_as_float(x[1]);  // lo: block 0, hi: block 2
  float q1 = __uint_as_float(y[0]) + __uint_as_float(y[1]);  // lo: block 1, hi: block 3
  // Step 2: within each half, row 0 keeps the first block and row 1 the second.
  // permlane16_swap(a, b) returns {[a_r0, b_r0], [a_r1, b_r1]} per 32-lane half.
  auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(q0), __float_as_uint(q1), false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// Direct-to-LDS loads (global_load_lds_dword / _dwordx4): lane l's bytes land at
// lds + size * l.  Issued through asm so that the compiler neither tracks their LDS
// writes (it would otherwise wait for them before unrelated LDS reads of the other
// buffer) nor counts them; the kernel waits for them explicitly with s_waitcnt vmcnt(0).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}
__device__ __forceinline__ void dma_16(const void* gsrc, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(gsrc) : "memory");
}
// the same with an immediate byte offset added to the global address
template <int OFF>
__device__ __forceinline__ void dma_16o(const void* gsrc, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:%2" ::"s"(lds), "v"(gsrc), "n"(OFF)
               : "memory");
}
__device__ __forceinline__ void dma_4(const void* gsrc, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(gsrc) : "memory");
}

// s_waitcnt vmcnt(m) for the largest m <= n in [0, C] (n is wave-uniform); waiting for
// fewer outstanding loads than n is always safe.  Vector memory loads complete in issue
// order, so vmcnt(n) with n = the loads issued after a group means that group has landed
// (stores issued in between only raise the count, which waits longer).
template <int C>
__device__ __forceinline__ void wait_vm_at_most(int n) {
  if constexpr (C == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (n >= C) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C) : "memory");
    else wait_vm_at_most<C - 1>(n);
  }
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

}  // namespace dsa
