// Deterministic top-k over materialised score rows (gfx950).
//
// GLM-5.2 技术报告速览, section "IndexShare": keep the k highest indexer scores of each
// query; GLM-5 technical report, section 3.2: the top-k operator must be deterministic.
// One workgroup per row: an MSB-first radix select (8-bit digits, LDS histogram) finds
// the k-th largest order key theta and how many keys equal to theta are needed; a final
// pass in position order emits keys > theta and the first needed keys == theta, using
// wave ballots plus a cross-wave prefix, so the output is in ascending position order
// and identical from run to run.
#include "dsa_common.hpp"
#include "dsa_launch.hpp"
#include "../../include/dsa.h"

namespace dsa {

template <int BS>
__global__ __launch_bounds__(BS) void topk_rows_kernel(const float* __restrict__ scores, int64_t row_stride,
                                                       int n, const int32_t* __restrict__ n_valid,
                                                       int causal_Lq, int causal_Lk, int k,
                                                       int32_t* __restrict__ idx, float* __restrict__ vals) {
  constexpr int NWV = BS / 64;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel[2];
  __shared__ uint32_t wsum[NWV][2];
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv_id = tid >> 6;
  const float* x = scores + (size_t)row * row_stride;
  int nv = n;
  if (n_valid) nv = n_valid[row];
  else if (causal_Lq > 0) nv = causal_Lk - causal_Lq + (row % causal_Lq) + 1;
  nv = max(0, min(nv, n));
  int32_t* out = idx + (size_t)row * k;
  float* vout = vals ? vals + (size_t)row * k : nullptr;

  if (nv <= k) {
    for (int j = tid; j < k; j += BS) {
      out[j] = j < nv ? j : -1;
      if (vout) vout[j] = j < nv ? x[j] : -INFINITY;
    }
    return;
  }

  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int j = tid; j < 256; j += BS) hist[j] = 0;
    __syncthreads();
    for (int e = tid; e < nv; e += BS) {
      const uint32_t key = order_key(x[e]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wv_id == 0) {
      const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                     h3 = hist[4 * lane + 3];
      const uint32_t tot = h0 + h1 + h2 + h3;
      uint32_t S = tot;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_down(S, d);
        if (lane + d < 64) S += o;
      }
      const uint32_t above = S - tot;
      if (above < krem && S >= krem) {  // exactly one lane
        uint32_t c = above, d;
        if (c + h3 >= krem) d = 4 * lane + 3;
        else { c += h3;
          if (c + h2 >= krem) d = 4 * lane + 2;
          else { c += h2;
            if (c + h1 >= krem) d = 4 * lane + 1;
            else { c += h1; d = 4 * lane; } } }
        sel[0] = d;
        sel[1] = c;
      }
    }
    __syncthreads();
    prefix |= sel[0] << shift;
    pmask |= 255u << shift;
    krem -= sel[1];
    __syncthreads();
  }
  const uint32_t theta = prefix, need_eq = krem;

  uint32_t out_n = 0, eq_seen = 0;
  for (int base = 0; base < nv && out_n < (uint32_t)k; base += BS) {
    const int e = base + tid;
    const bool v = e < nv;
    const float xv = v ? x[e] : 0.f;
    const uint32_t key = v ? order_key(xv) : 0u;
    const bool gt = v && key > theta;
    const bool eq = v && key == theta;
    const uint64_t meq = ballot(eq);
    if (lane == 0) wsum[wv_id][0] = popc64(meq);
    __syncthreads();
    uint32_t eq_before = eq_seen + rank_below(meq), eq_tot = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const uint32_t c = wsum[w][0];
      if (w < wv_id) eq_before += c;
      eq_tot += c;
    }
    const bool take = gt || (eq && eq_before < need_eq);
    const uint64_t mt = ballot(take);
    if (lane == 0) wsum[wv_id][1] = popc64(mt);
    __syncthreads();
    uint32_t pos = out_n + rank_below(mt), t_tot = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const uint32_t c = wsum[w][1];
      if (w < wv_id) pos += c;
      t_tot += c;
    }
    if (take) {
      out[pos] = e;
      if (vout) vout[pos] = xv;
    }
    out_n += t_tot;
    eq_seen += eq_tot;
    __syncthreads();
  }
}

hipError_t launch_topk_rows(const float* scores, int64_t row_stride, int rows, int n,
                            const int32_t* n_valid, int causal_Lq, int causal_Lk, int k,
                            int32_t* idx, float* vals, hipStream_t s) {
  if (n >= 65536) topk_rows_kernel<1024><<<rows, 1024, 0, s>>>(scores, row_stride, n, n_valid, causal_Lq, causal_Lk, k, idx, vals);
  else topk_rows_kernel<512><<<rows, 512, 0, s>>>(scores, row_stride, n, n_valid, causal_Lq, causal_Lk, k, idx, vals);
  return hipGetLastError();
}

}  // namespace dsa
