// Per-token E4M3 quantization of the indexer operands (gfx950): the step that produces
// the fp8 q^I and k^I rows the indexer kernels read, and that appends a decode step's new
// k^I row to the cache.
//
// GLM-5.2 技术报告速览, section "IndexShare": the indexer uses ReLU rather than softmax
// to stay fast and FP8-friendly; GLM 5.2: Built for Long Horizon Tasks, section 5.2: the
// indexer has its own light W_Q^I / W_K^I and a per-layer index-key cache.  The pages fix
// neither the FP8 flavour nor the scale granularity; as everywhere in this library the
// format is OCP E4M3 with one fp32 scale per token: scale = amax / 448 (1 for an all-zero
// token) and code = round-to-nearest-even of x / scale, both divisions in IEEE single
// precision.
//
// One wave per token row: a pass for the row's largest magnitude, then a pass that
// divides, rounds and stores four codes per lane per step.
#include "dsa_common.hpp"
#include "dsa_launch.hpp"
#include "../../include/dsa.h"

namespace dsa {

namespace {

// E4M3 code of y, |y| <= 448, round to nearest even, sign kept (-0 -> 0x80).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sgn = (__float_as_uint(y) >> 24) & 0x80u;
  const float ay = fminf(fabsf(y), 448.f);
  uint32_t code;
  if (ay < 0.015625f) {                 // below 2^-6: subnormal steps of 2^-9 (8 steps = 2^-6)
    code = (uint32_t)rintf(ay * 512.f);
  } else {                              // round the fp32 mantissa to 3 bits, rebias 127 -> 7
    uint32_t u = __float_as_uint(ay);
    u += 0x7ffffu + ((u >> 20) & 1u);
    code = (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);
  }
  return sgn | code;
}

template <bool kBf16>
__device__ __forceinline__ void load4(const void* row, int e, float (&v)[4]) {
  if constexpr (kBf16) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(row) + e);
    v[0] = __uint_as_float(w.x << 16);
    v[1] = __uint_as_float(w.x & 0xffff0000u);
    v[2] = __uint_as_float(w.y << 16);
    v[3] = __uint_as_float(w.y & 0xffff0000u);
  } else {
    const float4 w = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(row) + e);
    v[0] = w.x;
    v[1] = w.y;
    v[2] = w.z;
    v[3] = w.w;
  }
}

template <bool kBf16>
__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const void* __restrict__ x, int rows, int row_elems,
                                                            int64_t x_stride, uint8_t* __restrict__ codes,
                                                            int64_t c_stride, float* __restrict__ scales,
                                                            int64_t s_stride) {
  const int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const void* xr = kBf16 ? static_cast<const void*>(static_cast<const uint16_t*>(x) + (size_t)row * x_stride)
                         : static_cast<const void*>(static_cast<const float*>(x) + (size_t)row * x_stride);
  float amax = 0.f;
  for (int e = 4 * lane; e < row_elems; e += 256) {
    float v[4];
    load4<kBf16>(xr, e, v);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = amax > 0.f ? amax / 448.f : 1.f;
  uint8_t* cr = codes + (size_t)row * c_stride;
  for (int e = 4 * lane; e < row_elems; e += 256) {
    float v[4];
    load4<kBf16>(xr, e, v);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= e4m3_code(v[i] / scale) << (8 * i);
    *reinterpret_cast<uint32_t*>(cr + e) = w;
  }
  if (lane == 0) scales[(size_t)row * s_stride] = scale;
}

}  // namespace

hipError_t launch_quantize_e4m3(const void* x, int x_dtype, int rows, int row_elems, int64_t x_stride,
                                uint8_t* codes, int64_t c_stride, float* scales, int64_t s_stride, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (x_dtype == DSA_BF16)
    quantize_e4m3_kernel<true><<<grid, 256, 0, s>>>(x, rows, row_elems, x_stride, codes, c_stride, scales, s_stride);
  else
    quantize_e4m3_kernel<false><<<grid, 256, 0, s>>>(x, rows, row_elems, x_stride, codes, c_stride, scales, s_stride);
  return hipGetLastError();
}

}  // namespace dsa
