// bf16 linear map for the indexer's projections, the step before the path (GLM 5.2: Built
// for Long Horizon Tasks, discussion section "DSA 与 IndexShare 的组合数据流": the indexer
// keeps its own light projections W_Q^I, W_K^I beside the MLA path; GLM-5.2 技术报告速览,
// section "IndexShare": per-head gating weights w^I):
//   y[M, N] (fp32) = x[M, K] (bf16) . w[N, K]^T (bf16),
// i.e. every output is one dot product of a row of x with a row of w (the layout of a
// linear layer's weight).  The fp32 result feeds the per-token E4M3 quantization.
//
// One workgroup of 256 threads computes a 128 x 128 block of y.  K advances in 64-column
// steps: the x and w tiles of the next step are loaded straight into the other LDS buffer
// (last read in the step before, which the step's barrier closed) while the current
// step's tiles are read, so each step costs one wait and one workgroup barrier.  Each wave
// owns a 64 x 64 quarter of the block: 4 x 4 MFMA 16x16x32 bf16 accumulators, two K
// sub-steps of 32 per tile.  LDS rows are 64 bf16 = eight 16-byte chunks, stored with the
// chunk index XOR-ed with (row & 7) so that the 16 rows one operand read touches start in
// different banks.
#include "dsa_common.hpp"
#include "dsa_launch.hpp"
#include "../../include/dsa.h"

namespace dsa {

namespace {
constexpr int kLinTile = 128;   // rows of x and rows of w per workgroup
constexpr int kLinK = 64;       // K columns per LDS step

__device__ __forceinline__ int lin_slot(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }
}  // namespace

__global__ __launch_bounds__(256) void linear_bf16_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                          const uint16_t* __restrict__ w, int64_t ldw, int M,
                                                          int N, int K, float* __restrict__ y, int64_t ldy) {
  __shared__ __attribute__((aligned(16))) bf16x8 lx[2][kLinTile * 8];
  __shared__ __attribute__((aligned(16))) bf16x8 lw[2][kLinTile * 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (LDS bases go to M0)
  const int m0 = blockIdx.y * kLinTile, n0 = blockIdx.x * kLinTile;
  const int wm = (wv >> 1) * 64, wn = (wv & 1) * 64;

  // 128 rows x 8 chunks per operand, moved by direct-to-LDS loads: wave wv's load u fills
  // LDS slots 64 (4u + wv) .. + 63 (eight rows), lane l the slot's row r and physical chunk
  // pc, reading the row's logical chunk pc ^ (r & 7) (the swizzle above).  Rows past M or N
  // re-read the last row; their results are never stored.
  auto issue = [&](int k0, int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int slot = 64 * (4 * u + wv) + lane, r = slot >> 3, pc = slot & 7, ch = pc ^ (r & 7);
      const int gm = min(m0 + r, M - 1), gn = min(n0 + r, N - 1);
      dma_16(x + (size_t)gm * ldx + k0 + ch * 8, lds_offset(&lx[buf][64 * (4 * u + wv)]));
      dma_16(w + (size_t)gn * ldw + k0 + ch * 8, lds_offset(&lw[buf][64 * (4 * u + wv)]));
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_steps = K / kLinK;
  issue(0, 0);
  for (int kt = 0; kt < n_steps; ++kt) {
    const int cur = kt & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this step's tiles have landed
    __syncthreads();                                     // ... for every wave; the other buffer is free
    if (kt + 1 < n_steps) issue((kt + 1) * kLinK, cur ^ 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // lane l: row l % 16 of each 16-row block, K chunk 4 ks + l / 16 (8 bf16)
      const int ch = 4 * ks + (lane >> 4);
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = lx[cur][lin_slot(wm + 16 * i + (lane & 15), ch)];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = lw[cur][lin_slot(wn + 16 * j + (lane & 15), ch)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16_16x16x32(a[i], b[j], acc[i][j]);
    }
  }

  // acc[i][j] lane l: rows wm + 16 i + 4 (l / 16) + q, column wn + 16 j + l % 16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + wn + 16 * j + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gm = m0 + wm + 16 * i + 4 * (lane >> 4) + q;
        if (gm < M && gn < N) y[(size_t)gm * ldy + gn] = acc[i][j][q];
      }
    }
}

hipError_t launch_linear_bf16(const void* x, int64_t ldx, const void* w, int64_t ldw, int M, int N, int K, float* y,
                              int64_t ldy, hipStream_t s) {
  const dim3 grid((N + kLinTile - 1) / kLinTile, (M + kLinTile - 1) / kLinTile);
  linear_bf16_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), ldx, static_cast<const uint16_t*>(w), ldw,
                                          M, N, K, y, ldy);
  return hipGetLastError();
}

}  // namespace dsa
