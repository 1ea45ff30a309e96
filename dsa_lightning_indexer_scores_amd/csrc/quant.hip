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
// Rows that fit in registers (up to 8192 values: 64 lanes x 16 or 32 pieces of 16 bytes)
// are read from memory once: every lane loads its pieces, the row's lanes agree on the
// largest magnitude, and the codes come from the values still held.  Other rows take one
// wave each and two passes over the row.
#include "dsa_common.hpp"
#include "dsa_launch.hpp"
#include "../../include/dsa.h"

namespace dsa {

namespace {

// E4M3 code of |y| <= 448 (round to nearest even), without the sign bit.
__device__ __forceinline__ uint32_t e4m3_magnitude(float y) {
  const float ay = fminf(fabsf(y), 448.f);
  uint32_t code;
  if (ay < 0.015625f) {                 // below 2^-6: subnormal steps of 2^-9 (8 steps = 2^-6)
    code = (uint32_t)rintf(ay * 512.f);
  } else {                              // round the fp32 mantissa to 3 bits, rebias 127 -> 7
    uint32_t u = __float_as_uint(ay);
    u += 0x7ffffu + ((u >> 20) & 1u);
    code = (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);
  }
  return code;
}

// E4M3 code of y, sign kept (-0 -> 0x80).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  return ((__float_as_uint(y) >> 24) & 0x80u) | e4m3_magnitude(y);
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

// Register-resident rows.  A row is n_pieces x 2^lpr_log2 pieces of 16 bytes (8 bf16 or 4
// fp32 values); lane sub of the row's 2^lpr_log2 lanes holds pieces c * 2^lpr_log2 + sub,
// so each load and store instruction covers contiguous bytes, and one wave takes
// 64 / 2^lpr_log2 rows.  The quotient x / scale is formed as RN(q0 + r y) with
// y = RN(1 / scale), q0 = RN(x y) and r = x - scale q0 (exact by fma): with a correctly
// rounded reciprocal this is the correctly rounded quotient (Markstein's theorem), so the
// codes are those of the IEEE division.  The sign comes from x (scale > 0), which keeps
// -0 -> 0x80.  The theorem needs the residual r exact, which holds unless x is subnormal;
// a subnormal x only matters (gives a nonzero code) when scale < 2^-116, so a wave with a
// row whose scale is below 2^-100 divides instead.
template <bool kBf16>
__global__ __launch_bounds__(256) void quantize_e4m3_rows_kernel(const void* __restrict__ x, int rows, int n_pieces,
                                                                 int lpr_log2, int64_t x_stride,
                                                                 uint8_t* __restrict__ codes, int64_t c_stride,
                                                                 float* __restrict__ scales, int64_t s_stride) {
  constexpr int kPer = kBf16 ? 8 : 4;          // values per 16-byte piece
  constexpr int kMaxPieces = kBf16 ? 16 : 32;   // 8192 values either way
  constexpr int kEsize = kBf16 ? 2 : 4;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t row = (wave << (6 - lpr_log2)) + (lane >> lpr_log2);
  const int lpr = 1 << lpr_log2;
  const int sub = lane & (lpr - 1);
  const bool valid = row < rows;
  const uint8_t* xr = static_cast<const uint8_t*>(x) + (valid ? row : 0) * x_stride * kEsize;
  i32x4 v[kMaxPieces];
#pragma unroll
  for (int c = 0; c < kMaxPieces; ++c)
    if (c < n_pieces && valid) v[c] = *reinterpret_cast<const i32x4*>(xr + (size_t)(c * lpr + sub) * 16);
  auto value = [&](int c, int e) -> float {
    if constexpr (kBf16) {
      const uint32_t w = (uint32_t)v[c][e >> 1];
      return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
      return __int_as_float(v[c][e]);
    }
  };
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxPieces; ++c)
    if (c < n_pieces && valid)
#pragma unroll
      for (int e = 0; e < kPer; ++e) amax = fmaxf(amax, fabsf(value(c, e)));
  for (int off = lpr >> 1; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = amax > 0.f ? amax / 448.f : 1.f;
  const float y = 1.f / scale;
  uint8_t* cr = codes + (valid ? row : 0) * c_stride;
  auto encode = [&](auto by_recip) {
#pragma unroll
    for (int c = 0; c < kMaxPieces; ++c) {
      if (c < n_pieces && valid) {
        uint32_t w[kPer / 4] = {};
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          const float xe = value(c, e);
          float q;
          if constexpr (decltype(by_recip)::value) {
            const float q0 = xe * y;
            q = fmaf(fmaf(-q0, scale, xe), y, q0);
          } else {
            q = xe / scale;
          }
          const uint32_t code = ((__float_as_uint(xe) >> 24) & 0x80u) | e4m3_magnitude(q);
          w[e >> 2] |= code << (8 * (e & 3));
        }
        uint8_t* dst = cr + (size_t)(c * lpr + sub) * kPer;
        if constexpr (kBf16) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
        else *reinterpret_cast<uint32_t*>(dst) = w[0];
      }
    }
  };
  if (ballot(valid && !(scale >= 0x1p-100f)) == 0) encode(std::true_type{});   // wave-uniform
  else encode(std::false_type{});
  if (valid && sub == 0) scales[row * s_stride] = scale;
}

}  // namespace

hipError_t launch_quantize_e4m3(const void* x, int x_dtype, int rows, int row_elems, int64_t x_stride,
                                uint8_t* codes, int64_t c_stride, float* scales, int64_t s_stride, hipStream_t s) {
  // register-resident path: pieces of 16 bytes, a power of two of them up to 64 lanes, or
  // whole waves of up to 16 pieces per lane; 16-byte aligned rows and whole-piece codes
  const bool bf = x_dtype == DSA_BF16;
  const int per = bf ? 8 : 4, esize = bf ? 2 : 4;
  auto aligned_to = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
  if (row_elems % per == 0 && aligned_to(x, 16) && (x_stride * esize) % 16 == 0 && aligned_to(codes, per) &&
      c_stride % per == 0) {
    const int pieces = row_elems / per;
    int lpr_log2 = -1, n_pieces = 0;
    if (pieces <= 64 && (pieces & (pieces - 1)) == 0) {
      lpr_log2 = __builtin_ctz((unsigned)pieces);
      n_pieces = 1;
    } else if (pieces % 64 == 0 && pieces / 64 <= (bf ? 16 : 32)) {
      lpr_log2 = 6;
      n_pieces = pieces / 64;
    }
    if (lpr_log2 >= 0) {
      const int64_t rows_per_wave = 64 >> lpr_log2;
      const int64_t waves = (rows + rows_per_wave - 1) / rows_per_wave;
      const dim3 g((unsigned)((waves + 3) / 4));
      if (bf)
        quantize_e4m3_rows_kernel<true><<<g, 256, 0, s>>>(x, rows, n_pieces, lpr_log2, x_stride, codes, c_stride,
                                                          scales, s_stride);
      else
        quantize_e4m3_rows_kernel<false><<<g, 256, 0, s>>>(x, rows, n_pieces, lpr_log2, x_stride, codes, c_stride,
                                                           scales, s_stride);
      return hipGetLastError();
    }
  }
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (x_dtype == DSA_BF16)
    quantize_e4m3_kernel<true><<<grid, 256, 0, s>>>(x, rows, row_elems, x_stride, codes, c_stride, scales, s_stride);
  else
    quantize_e4m3_kernel<false><<<grid, 256, 0, s>>>(x, rows, row_elems, x_stride, codes, c_stride, scales, s_stride);
  return hipGetLastError();
}

}  // namespace dsa
