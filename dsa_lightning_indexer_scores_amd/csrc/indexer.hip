// Lightning-indexer kernels for gfx950.
//
// Score (GLM-5.2 技术报告速览, section "IndexShare", indexer-score equation):
//   I[t, s] = sum_j w[t, j] * ReLU(q^I[t, j] . k^I[s]),  s <= t.
// The dot products are a dense contraction (rows = query heads, columns = keys,
// K = d_I = 128) and run on MFMA: bf16 16x16x32, or OCP-E4M3 16x16x128 where one
// instruction covers the whole d_I.  ReLU, the head weights and (fp8) the per-token
// scales are applied to the accumulators in registers: the positive scales commute
// with ReLU, so q_scale[t] is folded into w[t, :] and k_scale[s] multiplies the summed
// score once per (t, s).  A 4-way lane reduce-scatter then leaves lane l holding the
// score of key s0 + l of a 64-key tile.
//
// Top-k (same section: keep the k best keys; GLM-5 technical report section 3.2: the
// operator must be deterministic): the fused kernel never writes the score matrix.
// Each query row is owned by one wave, which keeps a candidate buffer (uint32 order
// key, position) in ascending position order and a threshold theta; a key is appended
// only if its order key is > theta (ties with theta lose to the earlier positions
// already held).  When the buffer nears capacity the wave radix-selects the k-th key,
// sets theta to it and compacts the buffer in place, keeping positions in order and
// the lowest positions among keys equal to theta.
#include <type_traits>
#include "dsa_common.hpp"
#include "dsa_launch.hpp"
#include "../../include/dsa.h"

namespace dsa {

constexpr int kTileKeys = 64;
constexpr int kPersistentGrid = 1024;  // fixed so that workspace sizes are pure host math

template <int DT> struct IdxTraits;
template <> struct IdxTraits<DSA_BF16> {
  static constexpr int kRowBytes = 256;   // d_I = 128 bf16
  static constexpr int kTokensPerWave = 1;
};
template <> struct IdxTraits<DSA_FP8_E4M3> {
  static constexpr int kRowBytes = 128;   // d_I = 128 E4M3
  static constexpr int kTokensPerWave = 2;
};



// Per-lane operand slice of one 16-row block of a d_I = 128 row, for lane group g = lane/16.
// FP8 (one 16x16x128 MFMA): bytes [16g, 16g + 16) and [64 + 16g, 80 + 16g).  BF16 (four
// 16x16x32 MFMAs, i = 0..3): bytes [64i + 16g, 64i + 16g + 16).  Either way the four lane
// groups of one load instruction read one whole 64-byte half of each of the 16 rows.  A
// (queries) and B (keys) use the same slices, so the MFMA pairs equal feature indices.
template <int DT> struct Op;
template <> struct Op<DSA_FP8_E4M3> { i32x8 v; };
template <> struct Op<DSA_BF16> { bf16x8 v[4]; };

template <int DT>
__device__ __forceinline__ Op<DT> load_op(const uint8_t* row, int g);
template <>
__device__ __forceinline__ Op<DSA_FP8_E4M3> load_op<DSA_FP8_E4M3>(const uint8_t* row, int g) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(row + 16 * g);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(row + 64 + 16 * g);
  Op<DSA_FP8_E4M3> o;
  o.v = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return o;
}
template <>
__device__ __forceinline__ Op<DSA_BF16> load_op<DSA_BF16>(const uint8_t* row, int g) {
  Op<DSA_BF16> o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o.v[i] = *reinterpret_cast<const bf16x8*>(row + 64 * i + 16 * g);
  return o;
}

// Key tiles sit in LDS unpadded; the 16-byte chunks of a row are XOR-swizzled so that
// the 16 rows one MFMA operand reads start in distinct banks.
template <int DT>
__device__ __forceinline__ int tile_chunk(int r, int c) {
  return DT == DSA_FP8_E4M3 ? (c ^ ((r >> 1) & 7)) : (c ^ (r & 15));
}
// B operand (16 keys x d_I) of lane (r16, g) from a swizzled LDS key tile.
template <int DT>
__device__ __forceinline__ Op<DT> load_op_tile(const uint8_t* tile, int row, int g);
template <>
__device__ __forceinline__ Op<DSA_FP8_E4M3> load_op_tile<DSA_FP8_E4M3>(const uint8_t* tile, int row, int g) {
  const uint8_t* r = tile + row * 128;
  const i32x4 lo = *reinterpret_cast<const i32x4*>(r + 16 * tile_chunk<DSA_FP8_E4M3>(row, g));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(r + 16 * tile_chunk<DSA_FP8_E4M3>(row, g + 4));
  Op<DSA_FP8_E4M3> o;
  o.v = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return o;
}
template <>
__device__ __forceinline__ Op<DSA_BF16> load_op_tile<DSA_BF16>(const uint8_t* tile, int row, int g) {
  const uint8_t* r = tile + row * 256;
  Op<DSA_BF16> o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o.v[i] = *reinterpret_cast<const bf16x8*>(r + 16 * tile_chunk<DSA_BF16>(row, 4 * i + g));
  return o;
}

template <int DT>
__device__ __forceinline__ f32x4 dot16(const Op<DT>& a, const Op<DT>& b);
template <>
__device__ __forceinline__ f32x4 dot16<DSA_FP8_E4M3>(const Op<DSA_FP8_E4M3>& a, const Op<DSA_FP8_E4M3>& b) {
  return mfma_fp8_16x16x128(a.v, b.v, f32x4{0.f, 0.f, 0.f, 0.f});
}
template <>
__device__ __forceinline__ f32x4 dot16<DSA_BF16>(const Op<DSA_BF16>& a, const Op<DSA_BF16>& b) {
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) c = mfma_bf16_16x16x32(a.v[i], b.v[i], c);
  return c;
}

// ReLU as one integer max of the bit pattern: a float with its sign bit set is a negative
// int32, and non-negative floats order like their bit patterns.  Equal to fmaxf(x, 0) for
// every non-NaN x (-0 gives +0); fmaxf itself costs a second instruction that quiets
// signalling NaNs first.
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Scores of TW tokens against a 64-key tile.  a[tt][hb]: token tt's heads
// 16hb..16hb+15; b[kb]: keys 16kb..16kb+15 of the tile; wv[tt][hb][i] = w'[16hb + 4g + i].
// Returns, in lane l of out[tt], sum_j w'_j ReLU(q_j . k_{s0+l}) (before the fp8 key
// scale).  Shared by the materialising and the fused kernels so both produce identical
// bits (each token's arithmetic does not depend on TW, nor on the issue order below).
//
// FP8: one 16x16x128 MFMA per (key block, token, head block), and its epilogue (four
// ReLUs and four FMAs, 32 VALU cycles against the MFMA's 32) is issued kLag MFMAs later,
// when its result has long landed, between two MFMAs: MFMA m, epilogue m - kLag,
// MFMA m + 1, ...  The order is held by empty asm statements: the B operand of MFMA m
// passes through one that also takes the accumulator of epilogue m - 1 - kLag, so that
// epilogue cannot sink below the MFMA.  BF16 (four chained MFMAs per dot product): dot
// products go in pairs whose MFMAs alternate, so each chain's next MFMA waits behind the
// other chain's instead of on its own result, and the epilogue of the pair kLagP = 2
// pairs back is issued between the pair's MFMA steps, four VALU per step (two components
// of one of its dot products), pinned the same way: the B operand of the step's first
// MFMA passes through an empty asm statement that takes the last epilogue result.  The
// per-element arithmetic and its order are those of the plain schedule (bit-identical
// scores); the 16K bf16 indexer + top-k ran 4% faster than with groups of sixteen MFMAs
// followed by their epilogues.
template <int DT, int HB, int TW>
__device__ __forceinline__ void tile_scores(const Op<DT> (&a)[TW][HB], const Op<DT> (&b)[4],
                                            const f32x4 (&wv)[TW][HB], float (&out)[TW]) {
  float p[TW][4];
  if constexpr (DT == DSA_FP8_E4M3) {
    constexpr int N = 4 * TW * HB;   // MFMAs, in (key block, token, head block) order
    constexpr int kLag = 3;
    f32x4 d[N];
    Op<DT> bl[4] = {b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int m = 0; m < N + kLag; ++m) {
      if (m < N) {
        const int kb = m / (TW * HB), tt = (m / HB) % TW, hb = m % HB;
        if (m > kLag) {
          const int e = m - 1 - kLag;
          asm volatile("" : "+v"(bl[kb].v) : "v"(p[(e / HB) % TW][e / (TW * HB)]));
        }
        d[m] = dot16<DT>(a[tt][hb], bl[kb]);
        asm volatile("" : "+v"(d[m]));
      }
      if (m >= kLag) {
        const int e = m - kLag;
        const int kb = e / (TW * HB), tt = (e / HB) % TW, hb = e % HB;
        float acc = hb == 0 ? 0.f : p[tt][kb];
        acc = fmaf(wv[tt][hb][0], relu_bits(d[e][0]), acc);
        acc = fmaf(wv[tt][hb][1], relu_bits(d[e][1]), acc);
        acc = fmaf(wv[tt][hb][2], relu_bits(d[e][2]), acc);
        acc = fmaf(wv[tt][hb][3], relu_bits(d[e][3]), acc);
        p[tt][kb] = acc;
      }
    }
  } else {
    constexpr int N = 4 * TW * HB;   // dot products, in (key block, token, head block) order
    constexpr int NP = (N + 1) / 2;  // pairs (2q, 2q + 1)
    constexpr int kLagP = 2;
    f32x4 d[N];
    Op<DT> bl[4] = {b[0], b[1], b[2], b[3]};
    float last = 0.f;
#pragma unroll
    for (int q = 0; q < NP + kLagP; ++q) {
      const int m0 = 2 * q, m1 = 2 * q + 1;
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (m0 < N) {
          const int kb0 = m0 / (TW * HB), tt0 = (m0 / HB) % TW, hb0 = m0 % HB;
          if (q > kLagP || (q == kLagP && i > 0)) asm volatile("" : "+v"(bl[kb0].v[i]) : "v"(last));
          c0 = mfma_bf16_16x16x32(a[tt0][hb0].v[i], bl[kb0].v[i], c0);
          asm volatile("" : "+v"(c0));
        }
        if (m1 < N) {
          const int kb1 = m1 / (TW * HB), tt1 = (m1 / HB) % TW, hb1 = m1 % HB;
          c1 = mfma_bf16_16x16x32(a[tt1][hb1].v[i], bl[kb1].v[i], c1);
          asm volatile("" : "+v"(c1));
        }
        // epilogue of pair q - kLagP: two components of one of its dot products per step
        const int qe = q - kLagP;
        const int e = 2 * qe + (i >> 1);
        if (qe >= 0 && e < N) {
          const int kb = e / (TW * HB), tt = (e / HB) % TW, hb = e % HB;
          const int c = 2 * (i & 1);
          float acc = (hb == 0 && c == 0) ? 0.f : p[tt][kb];
          acc = fmaf(wv[tt][hb][c], relu_bits(d[e][c]), acc);
          acc = fmaf(wv[tt][hb][c + 1], relu_bits(d[e][c + 1]), acc);
          p[tt][kb] = acc;
          last = acc;
        }
      }
      if (m0 < N) d[m0] = c0;
      if (m1 < N) d[m1] = c1;
    }
  }
#pragma unroll
  for (int tt = 0; tt < TW; ++tt) out[tt] = reduce_scatter4(p[tt][0], p[tt][1], p[tt][2], p[tt][3]);
}

template <int DT, int HB>
__device__ __forceinline__ float tile_score(const Op<DT> (&a)[HB], const Op<DT> (&b)[4],
                                            const f32x4 (&wv)[HB]) {
  const Op<DT>(&a1)[1][HB] = *reinterpret_cast<const Op<DT>(*)[1][HB]>(&a);
  const f32x4(&w1)[1][HB] = *reinterpret_cast<const f32x4(*)[1][HB]>(&wv);
  float out[1];
  tile_scores<DT, HB, 1>(a1, b, w1, out);
  return out[0];
}

// ---------------------------------------------------------------------------
// Materialised scores: one workgroup per (query row, chunk of keys); each wave scans
// every fourth 64-key tile of the chunk, reading k^I straight from HBM (no reuse).
// ---------------------------------------------------------------------------
// Keys per workgroup: chosen so that rows x chunks fills the resident workgroup slots
// (4 per CU on the 256 CUs of gfx950) about once, without a partial last wave of
// workgroups.  The plan depends only on the sizes, so the workspace it implies is pure host
// arithmetic and every call with the same sizes makes the same launches.
constexpr long long kResidentSlots = 4LL * 256;
static int rowscan_chunk(int rows, int Lk) {
  const long long target = kResidentSlots;
  long long per_row = (target + rows - 1) / rows;
  const long long max_chunks = (Lk + 255) / 256;
  if (per_row > max_chunks) per_row = max_chunks;
  if (per_row < 1) per_row = 1;
  const long long chunk = ((Lk + per_row - 1) / per_row + 63) / 64 * 64;
  return (int)chunk;
}

template <int DT, int HB>
__global__ __launch_bounds__(256) void indexer_rowscan_kernel(IndexerArgs a, float* __restrict__ scores,
                                                              int64_t stride, uint32_t* __restrict__ row_hist,
                                                              int chunk_keys) {
  __shared__ uint32_t lhist[kRowHistBins];
  constexpr int RB = IdxTraits<DT>::kRowBytes;
  const int n_chunks = (a.Lk + chunk_keys - 1) / chunk_keys;
  const int qrow = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x - qrow * n_chunks;
  const int b = qrow / a.Lq, i = qrow - b * a.Lq;
  const int p = a.Lk - a.Lq + i;
  const int lane = threadIdx.x & 63, wv_id = threadIdx.x >> 6, g = lane >> 4;
  const int s_begin = chunk * chunk_keys;
  const int s_end = min(a.Lk, s_begin + chunk_keys);
  float* out = scores + (size_t)qrow * stride;

  const uint8_t* qptr = reinterpret_cast<const uint8_t*>(a.q) + (size_t)qrow * a.H_I * RB;
  Op<DT> A[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) A[hb] = load_op<DT>(qptr + (size_t)(hb * 16 + (lane & 15)) * RB, g);
  const float qs = (DT == DSA_FP8_E4M3) ? a.q_scale[qrow] : 1.f;
  f32x4 W[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) W[hb][ii] = a.w[(size_t)qrow * a.H_I + hb * 16 + 4 * g + ii] * qs;

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k) + (size_t)b * a.Lk * RB;
  const float* ksc = (DT == DSA_FP8_E4M3) ? a.k_scale + (size_t)b * a.Lk : nullptr;
  if (row_hist) {
    for (int j = threadIdx.x; j < kRowHistBins; j += 256) lhist[j] = 0;
    __syncthreads();
  }
  const int s_first = s_begin + wv_id * kTileKeys;
  const int s_causal_end = min(s_end, p + 1);      // keys past this are -inf for this query
  constexpr int kStride = 4 * kTileKeys;           // the four waves interleave tiles
  // Key rows are clamped into [s_begin, last]: loads of tiles past the causal end or the
  // chunk re-read the last row (an L2 hit) instead of being skipped, so every step issues
  // the same loads and the wait counts stay exact.
  const int last = max(s_begin, s_causal_end - 1);
  const int n_tiles = s_first < s_end ? (s_end - s_first + kStride - 1) / kStride : 0;
  auto load_tile = [&](int t, Op<DT> (&Bk)[4], float& kscale) {
    const int s0 = s_first + t * kStride;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = min(s0 + kb * 16 + (lane & 15), last);
      Bk[kb] = load_op<DT>(kbase + (size_t)key * RB, g);
    }
    if (DT == DSA_FP8_E4M3) kscale = ksc[min(s0 + lane, last)];
  };
  // Two tiles in flight per wave, in three buffers that rotate by name (the loop is
  // unrolled three ways): tile t is scored from buffer t % 3 while the loads of tiles t+1
  // and t+2 are outstanding.  A rotation by register copies would make every iteration
  // wait for the loads it had just issued.
  Op<DT> B0[4], B1[4], B2[4];
  float k0 = 1.f, k1 = 1.f, k2 = 1.f;
  if (n_tiles > 0) {
    load_tile(0, B0, k0);
    load_tile(1, B1, k1);
  }
  // request tile t + 2 into Bl (whose previous tile is done), then score tile t from Bk
  auto step = [&](int t, const Op<DT> (&Bk)[4], float kk, Op<DT> (&Bl)[4], float& kl) {
    load_tile(t + 2, Bl, kl);
    if (t >= n_tiles) return;                      // wave-uniform
    const int s = s_first + t * kStride + lane;
    float val = tile_score<DT, HB>(A, Bk, W);
    if (DT == DSA_FP8_E4M3) val *= kk;
    const bool causal = s < s_causal_end;
    if (s < s_end) out[s] = causal ? val : -INFINITY;
    if (row_hist && causal) atomicAdd(&lhist[order_key(val) >> 21], 1u);
  };
  for (int t = 0; t < n_tiles; t += 3) {
    step(t, B0, k0, B2, k2);
    step(t + 1, B1, k1, B0, k0);
    step(t + 2, B2, k2, B1, k1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the last prefetches (unused)
  if (row_hist) {
    __syncthreads();
    uint32_t* rh = row_hist + (size_t)qrow * kRowHistBins;
    for (int j = threadIdx.x; j < kRowHistBins; j += 256)
      if (lhist[j]) atomicAdd(&rh[j], lhist[j]);
  }
}

// ---------------------------------------------------------------------------
// Few query rows (decode): one workgroup per (query row, chunk of keys) scores the chunk
// exactly as indexer_rowscan_kernel (same tile_score, so the same bits), but keeps the
// scores in LDS.  At the end it adds its top-11-bit histogram to the row's, finds the
// digit dc of its own k-th largest key (count(digit > dc) < k <= count(digit >= dc); 0
// when the chunk has at most k causal keys) and writes the entries with digit >= dc, in
// position order, to its list.  The row's k-th key is at least every chunk's k-th key,
// so the row's top-k entries all reach the lists, and only about k entries per chunk are
// written instead of the whole score row.
// ---------------------------------------------------------------------------
constexpr int kSelMaxChunk = 16384;   // keys per chunk: their scores fill 64 KB of LDS

// Digit of the krem-th largest entry of a 2048-bin LDS histogram, for 256 threads (8
// bins each); the caller guarantees that the histogram holds at least krem entries.
__device__ uint32_t block_digit256(const uint32_t* hist, uint32_t krem, uint32_t* sh) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t h[8], tot = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    h[j] = hist[8 * tid + j];
    tot += h[j];
  }
  // entries in the bins of higher threads: suffix sum over threads
  uint32_t incl = tot;   // inclusive suffix within the wave (lanes >= this one)
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_down(incl, d);
    if (lane + d < 64) incl += o;
  }
  if (lane == 0) sh[w] = incl;   // wave total
  __syncthreads();
  uint32_t above = incl - tot;
  for (int i = w + 1; i < 4; ++i) above += sh[i];
  if (above < krem && above + tot >= krem) {
    uint32_t c = above;
    int dd = 8 * tid;
    for (int j = 7; j >= 0; --j) {
      if (c + h[j] >= krem) { dd = 8 * tid + j; break; }
      c += h[j];
    }
    sh[4] = (uint32_t)dd;
  }
  __syncthreads();
  const uint32_t d = sh[4];
  __syncthreads();
  return d;
}

template <int DT, int HB>
__global__ __launch_bounds__(256) void indexer_chunksel_kernel(IndexerArgs a, int k, ChunkLists L) {
  __shared__ float lsc[kSelMaxChunk];
  __shared__ uint32_t lhist[kRowHistBins];
  __shared__ uint32_t sh[16];
  __shared__ int lpage[kSelMaxChunk / 64 + 1];     // paged: physical page of each chunk page
  constexpr int RB = IdxTraits<DT>::kRowBytes;
  const int qrow = blockIdx.x / L.n_chunks;
  const int chunk = blockIdx.x - qrow * L.n_chunks;
  const int b = qrow / a.Lq, i = qrow - b * a.Lq;
  const int p = chunk_lists_seq_len(L, b, a.Lk) - a.Lq + i;   // query position (< 0: no keys)
  const int tid = threadIdx.x, lane = tid & 63, wv_id = tid >> 6, g = lane >> 4;
  const int s_begin = chunk * L.chunk;
  const int s_end = min(a.Lk, s_begin + L.chunk);

  const uint8_t* qptr = reinterpret_cast<const uint8_t*>(a.q) + (size_t)qrow * a.H_I * RB;
  Op<DT> A[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) A[hb] = load_op<DT>(qptr + (size_t)(hb * 16 + (lane & 15)) * RB, g);
  const float qs = (DT == DSA_FP8_E4M3) ? a.q_scale[qrow] : 1.f;
  f32x4 W[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) W[hb][ii] = a.w[(size_t)qrow * a.H_I + hb * 16 + 4 * g + ii] * qs;

  const bool paged = L.block_table != nullptr;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k) + (paged ? 0 : (size_t)b * a.Lk * RB);
  const float* ksc = (DT == DSA_FP8_E4M3) ? a.k_scale + (paged ? 0 : (size_t)b * a.Lk) : nullptr;
  for (int j = tid; j < kRowHistBins; j += 256) lhist[j] = 0;

  const int s_first = s_begin + wv_id * kTileKeys;
  const int s_causal_end = min(s_end, p + 1);      // keys past this are not candidates
  constexpr int kStride = 4 * kTileKeys;           // the four waves interleave tiles
  // key rows clamped into [s_begin, last] (see indexer_rowscan_kernel)
  const int last = max(s_begin, s_causal_end - 1);
  const int n_tiles = s_first < s_causal_end ? (s_causal_end - s_first + kStride - 1) / kStride : 0;
  // paged: the physical pages of the chunk's positions [s_begin, last] go to LDS once
  const int pg0 = s_begin >> L.page_log2;
  if (paged && s_begin < s_causal_end) {
    const int n_pg = (last >> L.page_log2) - pg0 + 1;
    for (int j = tid; j < n_pg; j += 256) {
      const int pg = L.block_table[(size_t)b * L.max_pages + pg0 + j];
      lpage[j] = min(max(pg, 0), L.pool_pages - 1);
    }
  }
  __syncthreads();
  // A 64-key tile lies in one page (pages are multiples of 64 keys, tiles 64-aligned, and
  // clamped keys stay in the page of min(tile start, last)): one LDS lookup per tile.
  auto load_tile = [&](int t, Op<DT> (&Bk)[4], float& kscale) {
    const int s0 = s_first + t * kStride;
    int64_t shift = 0;                               // physical row - position, this tile
    if (paged) {
      const int kt = min(s0, last);
      const int lp = kt >> L.page_log2;
      shift = ((int64_t)lpage[lp - pg0] - lp) << L.page_log2;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = min(s0 + kb * 16 + (lane & 15), last);
      Bk[kb] = load_op<DT>(kbase + (size_t)(key + shift) * RB, g);
    }
    if (DT == DSA_FP8_E4M3) kscale = ksc[(size_t)(min(s0 + lane, last) + shift)];
  };
  // two tiles in flight in three buffers rotating by name (see indexer_rowscan_kernel)
  Op<DT> B0[4], B1[4], B2[4];
  float k0 = 1.f, k1 = 1.f, k2 = 1.f;
  if (n_tiles > 0) {
    load_tile(0, B0, k0);
    load_tile(1, B1, k1);
  }
  auto step = [&](int t, const Op<DT> (&Bk)[4], float kk, Op<DT> (&Bl)[4], float& kl) {
    load_tile(t + 2, Bl, kl);
    if (t >= n_tiles) return;                      // wave-uniform
    const int s = s_first + t * kStride + lane;
    float val = tile_score<DT, HB>(A, Bk, W);
    if (DT == DSA_FP8_E4M3) val *= kk;
    if (s < s_causal_end) {
      lsc[s - s_begin] = val;
      atomicAdd(&lhist[order_key(val) >> 21], 1u);
    }
  };
  for (int t = 0; t < n_tiles; t += 3) {
    step(t, B0, k0, B2, k2);
    step(t + 1, B1, k1, B0, k0);
    step(t + 2, B2, k2, B1, k1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the last prefetches (unused)
  __syncthreads();

  uint32_t* rh = L.row_hist + (size_t)qrow * kRowHistBins;
  for (int j = tid; j < kRowHistBins; j += 256)
    if (lhist[j]) atomicAdd(&rh[j], lhist[j]);
  const int n_c = max(0, s_causal_end - s_begin);
  const uint32_t dc = n_c > k ? block_digit256(lhist, (uint32_t)k, sh) : 0u;

  // Ordered compaction of the entries with digit >= dc.  Wave w takes the contiguous
  // range [w q, min(n_c, (w + 1) q)) of the chunk (q = n_c / 4 rounded up to 64, at most
  // 64 entries per lane), holds its keys in registers and counts its entries; after a
  // barrier it writes them behind those of the lower waves, in position order (ballot
  // rank), into the score buffer itself (keys at [0, n), chunk offsets at [8192, 8192 + n));
  // the workgroup then copies both arrays out in full 16-byte pieces.  More than 8192
  // entries (heavy ties) go straight to global memory instead.
  const size_t slot = (size_t)qrow * L.row_stride + (size_t)chunk * L.chunk;
  uint32_t* ok = L.keys + slot;
  uint32_t* op = L.pos + slot;
  constexpr int kHalf = kSelMaxChunk / 2;
  const int q = (n_c + 255) / 256 * 64;
  const int lo = min(n_c, wv_id * q), hi = min(n_c, lo + q);
  uint32_t kr[kSelMaxChunk / 256];
  uint32_t n_w = 0;
#pragma unroll
  for (int i = 0; i < kSelMaxChunk / 256; ++i) {
    const int e = lo + 64 * i + lane;
    kr[i] = e < hi ? order_key(lsc[e]) : 0u;
    n_w += (uint32_t)popc64(ballot(e < hi && (kr[i] >> 21) >= dc));
  }
  if (lane == 0) sh[8 + wv_id] = n_w;   // block_digit256 uses sh[0..4]
  __syncthreads();                      // every wave holds its keys: lsc may be overwritten
  uint32_t base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t c = sh[8 + w];
    base += w < wv_id ? c : 0u;
    total += c;
  }
  const bool staged = total <= (uint32_t)kHalf;   // workgroup-uniform
  uint32_t* lk = reinterpret_cast<uint32_t*>(lsc);
#pragma unroll
  for (int i = 0; i < kSelMaxChunk / 256; ++i) {
    const int e = lo + 64 * i + lane;
    const bool take = e < hi && (kr[i] >> 21) >= dc;
    const uint64_t m = ballot(take);
    if (take) {
      const uint32_t o = base + rank_below(m);
      if (staged) {
        lk[o] = kr[i];
        lk[kHalf + o] = (uint32_t)e;
      } else {
        ok[o] = kr[i];
        op[o] = (uint32_t)(s_begin + e);
      }
    }
    base += (uint32_t)popc64(m);
  }
  if (staged) {
    __syncthreads();
    for (uint32_t j = 4 * tid; j < total; j += 1024) {
      if (j + 4 <= total) {
        *reinterpret_cast<i32x4*>(ok + j) = *reinterpret_cast<const i32x4*>(lk + j);
        i32x4 p4 = *reinterpret_cast<const i32x4*>(lk + kHalf + j);
        p4 += s_begin;
        *reinterpret_cast<i32x4*>(op + j) = p4;
      } else {
        for (uint32_t jj = j; jj < total; ++jj) {
          ok[jj] = lk[jj];
          op[jj] = (uint32_t)s_begin + lk[kHalf + jj];
        }
      }
    }
  }
  if (tid == 0) L.cnt[(size_t)qrow * L.n_chunks + chunk] = total;
}

// After every chunk of a row is scored: one workgroup per (chunk, row) finds the row's
// k-th digit d1 from its histogram (the same rule as the row selection) and compacts the
// chunk's list in place to its entries of digit >= d1, keeping their order (an entry
// only moves to a lower slot, and a batch is read before any of it is written).
__global__ __launch_bounds__(256) void lists_filter_kernel(ChunkLists L, int causal_Lq, int causal_Lk, int k) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kRowHistBins];
  __shared__ uint32_t sh[8 * 4];
  const int row = blockIdx.y, c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nv = chunk_lists_seq_len(L, row / causal_Lq, causal_Lk) - causal_Lq + (row % causal_Lq) + 1;
  if (nv <= k) return;                                  // short rows need no lists
  const i32x4* rh = reinterpret_cast<const i32x4*>(L.row_hist + (size_t)row * kRowHistBins);
  const i32x4 h0 = rh[2 * tid], h1 = rh[2 * tid + 1];
  reinterpret_cast<i32x4*>(hist)[2 * tid] = h0;
  reinterpret_cast<i32x4*>(hist)[2 * tid + 1] = h1;
  __syncthreads();
  const uint32_t d1 = block_digit256(hist, (uint32_t)k, sh);
  uint32_t* cnt = L.cnt + (size_t)row * L.n_chunks + c;
  const uint32_t m = *cnt;
  const size_t base = (size_t)row * L.row_stride + (size_t)c * L.chunk;
  uint32_t* keys = L.keys + base;
  uint32_t* pos = L.pos + base;
  constexpr int kU = 8;
  uint32_t out_n = 0;
  for (uint32_t j0 = 0; j0 < m; j0 += kU * 256) {
    uint32_t key[kU], ps[kU];
    uint64_t msk[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t j = j0 + 256 * u + tid;
      key[u] = j < m ? keys[j] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t j = j0 + 256 * u + tid;
      const bool take = j < m && (key[u] >> 21) >= d1;
      ps[u] = take ? pos[j] : 0u;
      msk[u] = ballot(take);
    }
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < kU; ++u) sh[4 * u + w] = (uint32_t)popc64(msk[u]);
    }
    __syncthreads();                                   // the whole batch has been read
    uint32_t before[kU], run = 0;
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        if (ww == w) before[u] = run;
        run += sh[4 * u + ww];
      }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if ((msk[u] >> lane) & 1ull) {
        const uint32_t o = out_n + before[u] + rank_below(msk[u]);
        keys[o] = key[u];
        pos[o] = ps[u];
      }
    }
    out_n += run;
    __syncthreads();                                   // sh reused by the next batch
  }
  if (tid == 0) *cnt = out_n;
}

// Reference-size fp32 path: one thread per (query, key); q row and weights in LDS.
__global__ __launch_bounds__(256) void indexer_f32_kernel(IndexerArgs a, float* __restrict__ scores, int64_t stride,
                                                          uint32_t* __restrict__ row_hist) {
  extern __shared__ float smem[];
  const int n_chunks = (a.Lk + 255) / 256;
  const int qrow = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x - qrow * n_chunks;
  const int b = qrow / a.Lq, i = qrow - b * a.Lq;
  const int p = a.Lk - a.Lq + i;
  const int HD = a.H_I * a.d_I;
  float* qs = smem;
  float* ws = smem + HD;
  const float* q = reinterpret_cast<const float*>(a.q) + (size_t)qrow * HD;
  for (int e = threadIdx.x; e < HD; e += blockDim.x) qs[e] = q[e];
  for (int e = threadIdx.x; e < a.H_I; e += blockDim.x) ws[e] = a.w[(size_t)qrow * a.H_I + e];
  __syncthreads();
  const int s = chunk * 256 + threadIdx.x;
  if (s >= a.Lk) return;
  float val = -INFINITY;
  if (s <= p) {
    const float* kr = reinterpret_cast<const float*>(a.k) + ((size_t)b * a.Lk + s) * a.d_I;
    float acc = 0.f;
    for (int j = 0; j < a.H_I; ++j) {
      float d = 0.f;
      for (int e = 0; e < a.d_I; ++e) d = fmaf(qs[j * a.d_I + e], kr[e], d);
      acc = fmaf(ws[j], fmaxf(d, 0.f), acc);
    }
    val = acc;
    if (row_hist) atomicAdd(&row_hist[(size_t)qrow * kRowHistBins + (order_key(val) >> 21)], 1u);
  }
  scores[(size_t)qrow * stride + s] = val;
}

// ---------------------------------------------------------------------------
// Wave-level selection on a candidate list held as two arrays in global memory:
// keys[0..n) (uint32 order keys) and pos[0..n) (positions, ascending).  One pass reads
// the list in batches of 1024 entries: lane l holds entries base + 256 j + 4 l + i
// (j, i = 0..3), loaded as 16-byte vectors, and the next batch is requested before the
// current one is processed, so each pass costs about one memory latency per batch.
// ---------------------------------------------------------------------------
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;          // 2048 LDS bins per wave
constexpr int kBinsPerLane = kBins / 64;
constexpr uint32_t kBatch = 1024;

__device__ __forceinline__ void load_batch(const uint32_t* v, uint32_t base, uint32_t n, uint32_t (&x)[16]) {
  const uint32_t l4 = 4u * lane_id();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t e = base + 256u * j + l4;
    if (e + 3 < n) {
      const uint4 t = *reinterpret_cast<const uint4*>(v + e);
      x[4 * j] = t.x; x[4 * j + 1] = t.y; x[4 * j + 2] = t.z; x[4 * j + 3] = t.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * j + i] = (e + i < n) ? v[e + i] : 0u;
    }
  }
}

// Histogram of bits [shift, shift + nbits) of the keys whose higher bits equal prefix.
// keys must be 16-byte aligned.
__device__ void hist_pass(const uint32_t* keys, uint32_t n, uint32_t prefix, uint32_t pmask, int shift,
                          int nbits, uint32_t* hist) {
  const int lane = lane_id();
  const uint32_t dmask = (1u << nbits) - 1u;
  for (int b = lane; b < kBins; b += 64) hist[b] = 0;
  wave_lds_fence();
  uint32_t cur[16], nxt[16];
  if (n > 0) load_batch(keys, 0, n, cur);
  for (uint32_t base = 0; base < n; base += kBatch) {
    if (base + kBatch < n) load_batch(keys, base + kBatch, n, nxt);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t e = base + 256u * (q >> 2) + 4u * lane + (q & 3);
      if (e < n && (cur[q] & pmask) == prefix) atomicAdd(&hist[(cur[q] >> shift) & dmask], 1u);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) cur[q] = nxt[q];
  }
  wave_lds_fence();
}

// Digit d of the krem-th largest key: count(digit > d) < krem <= count(digit >= d).
// Returns d, above = count(digit > d) and at = count(digit == d).
__device__ void find_digit(const uint32_t* hist, uint32_t krem, uint32_t& d, uint32_t& above, uint32_t& at) {
  const int lane = lane_id();
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < kBinsPerLane; ++j) tot += hist[lane * kBinsPerLane + j];
  uint32_t S = tot;  // inclusive suffix sum over lanes >= this lane
#pragma unroll
  for (int dd = 1; dd < 64; dd <<= 1) {
    const uint32_t o = __shfl_down(S, dd);
    if (lane + dd < 64) S += o;
  }
  const uint32_t above_lane = S - tot;
  const bool here = (above_lane < krem) && (S >= krem);
  const int src = __ffsll((long long)ballot(here)) - 1;
  uint32_t c = above_lane, dig = 0, h = 0;
  for (int j = kBinsPerLane - 1; j >= 0; --j) {
    h = hist[lane * kBinsPerLane + j];
    dig = lane * kBinsPerLane + j;
    if (c + h >= krem) break;
    c += h;
  }
  d = __shfl(dig, src);
  above = __shfl(c, src);
  at = __shfl(h, src);
  wave_lds_fence();
}

// Exclusive prefix over lanes of a per-lane count c in 0..7, and the wave total.
__device__ __forceinline__ uint32_t lane_prefix(uint32_t c, uint32_t& total) {
  const uint64_t b0 = ballot(c & 1u), b1 = ballot(c & 2u), b2 = ballot(c & 4u);
  total = popc64(b0) + 2u * popc64(b1) + 4u * popc64(b2);
  return rank_below(b0) + 2u * rank_below(b1) + 4u * rank_below(b2);
}

// Stable compaction of the entries with take(key, eq, eq_rank) true, where eq_rank is the
// number of keys == theta that precede the entry: put(dst, key, pos) receives the kept
// entries at dst = 0, 1, ... in list order.  Destinations never pass the entries still to
// be read (dst <= index), so put may write the list itself (in-place compaction).
template <typename Take, typename Put>
__device__ uint32_t compact_list(const uint32_t* keys, const uint32_t* pos, uint32_t n, uint32_t theta, Take take,
                                 Put put) {
  const int lane = lane_id();
  uint32_t out = 0, eq_seen = 0;
  uint32_t ck[16], cp[16], nk[16], np[16];
  if (n > 0) { load_batch(keys, 0, n, ck); load_batch(pos, 0, n, cp); }
  for (uint32_t base = 0; base < n; base += kBatch) {
    if (base + kBatch < n) { load_batch(keys, base + kBatch, n, nk); load_batch(pos, base + kBatch, n, np); }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t e0 = base + 256u * j + 4u * lane;
      uint32_t eqc = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) eqc += (e0 + i < n && ck[4 * j + i] == theta) ? 1u : 0u;
      uint32_t eq_tot;
      uint32_t eq_r = eq_seen + lane_prefix(eqc, eq_tot);
      bool tk[4];
      uint32_t tc = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v = e0 + i < n;
        const bool eq = v && ck[4 * j + i] == theta;
        tk[i] = v && take(ck[4 * j + i], eq, eq_r);
        eq_r += eq ? 1u : 0u;
        tc += tk[i] ? 1u : 0u;
      }
      uint32_t t_tot;
      uint32_t dst = out + lane_prefix(tc, t_tot);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tk[i]) {
          put(dst, ck[4 * j + i], cp[4 * j + i]);
          ++dst;
        }
      out += t_tot;
      eq_seen += eq_tot;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) { ck[q] = nk[q]; cp[q] = np[q]; }
  }
  return out;
}

// Exact k-th largest key theta among keys[0..n) (n > k) and need_eq, the number of
// entries equal to theta in the top k (the first need_eq of them in array order).
__device__ void select_exact(const uint32_t* keys, uint32_t n, uint32_t k, uint32_t* hist, uint32_t& theta,
                             uint32_t& need_eq) {
  uint32_t prefix = 0, pmask = 0, krem = k, d, above, at;
  hist_pass(keys, n, prefix, pmask, 21, 11, hist);
  find_digit(hist, krem, d, above, at);
  prefix = d << 21; pmask = 0x7FFu << 21; krem -= above;
  hist_pass(keys, n, prefix, pmask, 10, 11, hist);
  find_digit(hist, krem, d, above, at);
  prefix |= d << 10; pmask |= 0x7FFu << 10; krem -= above;
  hist_pass(keys, n, prefix, pmask, 0, 10, hist);
  find_digit(hist, krem, d, above, at);
  theta = prefix | d;
  need_eq = krem - above;
}

// Stable compaction keeping keys > theta and the first need_eq keys == theta, in place or
// into separate arrays (put).
template <typename Put>
__device__ uint32_t compact_exact_to(const uint32_t* keys, const uint32_t* pos, uint32_t n, uint32_t theta,
                                     uint32_t need_eq, Put put) {
  return compact_list(keys, pos, n, theta, [=](uint32_t key, bool eq, uint32_t eq_rank) {
    return key > theta || (eq && eq_rank < need_eq);
  }, put);
}
__device__ uint32_t compact_exact(uint32_t* keys, uint32_t* pos, uint32_t n, uint32_t theta, uint32_t need_eq) {
  return compact_exact_to(keys, pos, n, theta, need_eq, [=](uint32_t d, uint32_t key, uint32_t p) {
    keys[d] = key;
    pos[d] = p;
  });
}

// In-place stable compaction keeping every key >= th.
__device__ uint32_t compact_ge(uint32_t* keys, uint32_t* pos, uint32_t n, uint32_t th) {
  return compact_list(keys, pos, n, th, [=](uint32_t key, bool, uint32_t) { return key >= th; },
                      [=](uint32_t d, uint32_t key, uint32_t p) {
                        keys[d] = key;
                        pos[d] = p;
                      });
}

// Exact top-k of a candidate list: afterwards keys/pos[0..min(n,k)) hold the k largest
// keys (ties to the earlier entry), in their original order.  kth receives the k-th
// largest key when the list held more than k entries, else 0.
__device__ uint32_t reduce_to_k(uint32_t* keys, uint32_t* pos, uint32_t n, uint32_t k, uint32_t* hist,
                                uint32_t& kth) {
  kth = 0u;
  if (n <= k) return n;
  __threadfence_block();
  uint32_t th, ne;
  select_exact(keys, n, k, hist, th, ne);
  kth = th;
  const uint32_t r = compact_exact(keys, pos, n, th, ne);
  __threadfence_block();
  return r;
}

// Exact top-k of a candidate list, written straight to its destination: put(j, key, pos)
// receives the kept entries j = 0 .. min(n, k) - 1 in list order (the k largest keys, ties
// to the earlier entry); the list itself is not modified.  Returns min(n, k).
template <typename Put>
__device__ uint32_t select_to(const uint32_t* keys, const uint32_t* pos, uint32_t n, uint32_t k, uint32_t* hist,
                              Put put) {
  __threadfence_block();   // the wave's own list stores are visible to its loads
  if (n <= k) {
    for (uint32_t j = (uint32_t)lane_id(); j < n; j += 64) put(j, keys[j], pos[j]);
    return n;
  }
  uint32_t th, ne;
  select_exact(keys, n, k, hist, th, ne);
  return compact_exact_to(keys, pos, n, th, ne, put);
}

// Make room in a streaming candidate list that holds n > k entries: drop every key below
// a lower bound of the k-th largest key.  The bound is the lower edge of the 22-bit key
// prefix that contains the k-th largest key (two histogram passes, one filtering pass);
// when that prefix holds too many keys the exact selection is used.  Returns the new
// count; theta receives the bound (the streaming filter then admits keys > theta: the
// list keeps at least k keys >= theta that precede any later one, so a later key equal
// to theta cannot enter the top k).
__device__ uint32_t shrink_list(uint32_t* keys, uint32_t* pos, uint32_t n, uint32_t k, uint32_t keep_max,
                                uint32_t* hist, uint32_t& theta) {
  __threadfence_block();
  uint32_t d1, a1, h1, d2, a2, h2;
  hist_pass(keys, n, 0u, 0u, 21, 11, hist);
  find_digit(hist, k, d1, a1, h1);
  hist_pass(keys, n, d1 << 21, 0x7FFu << 21, 10, 11, hist);
  find_digit(hist, k - a1, d2, a2, h2);
  uint32_t r;
  if (a1 + a2 + h2 <= keep_max) {
    theta = (d1 << 21) | (d2 << 10);
    r = compact_ge(keys, pos, n, theta);
  } else {
    uint32_t prefix = (d1 << 21) | (d2 << 10), krem = k - a1 - a2, d3, a3, h3;
    hist_pass(keys, n, prefix, 0x3FFFFFu << 10, 0, 10, hist);
    find_digit(hist, krem, d3, a3, h3);
    theta = prefix | d3;
    r = compact_exact(keys, pos, n, theta, krem - a3);
  }
  __threadfence_block();
  return r;
}

// ---------------------------------------------------------------------------
// Fused streaming indexer + top-k (persistent workgroups, atomic work queue).
// Work item = (sequence, block of TQ consecutive queries, key segment); blocks with the
// most causal keys are dispatched first.  With one segment the kernel writes idx
// directly; with several it writes each segment's top-k list for a merge kernel.
// ---------------------------------------------------------------------------
constexpr int kStage = 256;   // staged candidates per token before a bulk append

// Appends the n <= kStage staged candidates (LDS, in position order; each the score's
// float bits and its position) to the global list after its cnt entries, as order keys;
// returns the new count.  All reads are issued before the first store.
__device__ uint32_t flush_stage(const uint2* st, uint32_t n, uint32_t* keys, uint32_t* pos, uint32_t cnt) {
  const uint32_t lane = (uint32_t)lane_id();
  wave_lds_fence();
  uint2 e[kStage / 64];
#pragma unroll
  for (int u = 0; u < kStage / 64; ++u)
    if (lane + 64u * u < n) e[u] = st[lane + 64u * u];
#pragma unroll
  for (int u = 0; u < kStage / 64; ++u) {
    const uint32_t j = lane + 64u * u;
    if (j < n) {
      keys[cnt + j] = order_key(__uint_as_float(e[u].x));
      pos[cnt + j] = e[u].y;
    }
  }
  wave_lds_fence();  // the stage is refilled only after these reads
  return cnt + n;
}

// Speculative starting threshold.  Before its main pass, an item scores a sample of
// kSampleTiles key tiles spread over the keys that are causal for all its tokens, and each
// token starts its filter at the j-th largest of its m = 64 kSampleTiles sample keys
// instead of admitting every key, with j = mu + z sqrt(mu) + 1 and mu = m k / n the number
// of sample keys expected above the k-th of the token's n causal keys (about twice k keys
// then pass it); z = 4, or 6 with key segments.  Whatever the threshold, if at least k keys of a row pass it, the row's
// k-th largest key passes it, so the exact selection over the admitted keys is the row's
// top-k (ties included).  With one key segment per row, a row that admits fewer than
// min(k, its causal keys) sends its item to a second launch, which recomputes the item's
// rows without speculation.  With several key segments, a row's segments are separate
// items started from different thresholds; the merge takes the largest of them, Theta, and
// accepts the row only if at least min(k, its causal keys) of its list entries exceed
// Theta (then the row's k-th key exceeds every segment's threshold, so each top-k key was
// admitted in its segment); otherwise it sends every segment item of the row's query
// block to the second launch.  Rows with fewer than kSpecMinKeys causal keys, and items
// whose common causal keys span fewer than kSampleMinSpan, never speculate.
constexpr int kSpecMinKeys = 8192;
constexpr int kSampleTiles = 16;
constexpr int kSampleMinSpan = 4 * kSampleTiles * 64;

struct FusedParams {
  IndexerArgs a;
  int k, cap, S, seg_len, nqb, n_items;
  int pass;             // 0: every item, speculative thresholds; 1: the failed items, exact
  int* fail_count;      // items recorded by pass 0
  int* fail_items;      // [n_items * 8]: one entry per failing token (repeats are harmless)
  int* counter2;        // work counter of pass 1
  uint32_t* seg_spec;   // [B * Lq * S] starting threshold (order key, 0: none) of each segment (S > 1)
  int32_t* idx;
  uint32_t* row_keys;   // [grid * TQ * cap]
  uint32_t* row_pos;
  int seg_stride;       // entries per row of the segment lists (S * k rounded up to 4)
  uint32_t* seg_keys;   // [B * Lq * seg_stride]   (S > 1)
  uint32_t* seg_pos;
  int32_t* seg_cnt;     // [B * Lq * S]
  int* counter;         // work counters (the launch zeroes 16 ints)
};

template <int DT, int HB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void indexer_topk_kernel(FusedParams P) {
  constexpr int RB = IdxTraits<DT>::kRowBytes;
  constexpr int TW = IdxTraits<DT>::kTokensPerWave;
  constexpr int TQ = 4 * TW;
  constexpr int H_I = HB * 16;
  constexpr int kChunks = RB / 16;                 // 16-byte chunks per key row
  constexpr int kTileBytes = kTileKeys * RB;
  constexpr int kDmaPerWave = kTileBytes / 1024 / 4;
  // Key tile ring: tile t is scored from buffer t % kBufs while the next kBufs - 1 tiles
  // load.  Three buffers (two tiles in flight) for fp8 keys; bf16 tiles are twice the
  // size and keep two, which leaves room for two workgroups per CU.
  constexpr int kBufs = (DT == DSA_FP8_E4M3) ? 3 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t ktile[kBufs][kTileBytes];
  __shared__ __attribute__((aligned(16))) float kscl[kBufs][kTileKeys];
  __shared__ __attribute__((aligned(16))) float wsh[TQ * H_I];
  __shared__ uint32_t hist[4][kBins];
  // per-token staging of admitted candidates (score bits, position): appends are LDS
  // writes, and the global list receives them in bulk, as order keys (tile loads then
  // never wait for candidate stores)
  __shared__ __attribute__((aligned(8))) uint2 stg[TQ][kStage];
  __shared__ int item_sh;

  const IndexerArgs& a = P.a;
  const int lane = threadIdx.x & 63, g = lane >> 4;
  const int wv_id = uniform((int)(threadIdx.x >> 6));
  const bool fp8 = (DT == DSA_FP8_E4M3);

  for (;;) {
    __syncthreads();   // every wave is done with the previous item (its k-th keys recorded)
    if (threadIdx.x == 0) {
      int it;
      if (P.pass == 0 && P.S > 1) {
        // XCD-local queues: the items, ordered by (segment, query block), are cut into
        // eight ranges, and a workgroup takes items from the range of its XCD (workgroups
        // are dealt to the eight XCDs round-robin), so the workgroups sharing an L2 stream
        // the same segment's keys together; an exhausted range sends it to the others.
        const int rows_s = P.n_items / P.S;
        it = P.n_items;
        for (int v = 0; v < 8; ++v) {
          const int x = (int)((blockIdx.x + v) & 7);
          const int lo = (int)((long long)P.n_items * x / 8), hi = (int)((long long)P.n_items * (x + 1) / 8);
          const int j = atomicAdd(P.counter + 8 + x, 1);
          if (lo + j < hi) {
            const int i = lo + j;
            it = (i % rows_s) * P.S + i / rows_s;
            break;
          }
        }
      } else if (P.pass == 0) {
        it = atomicAdd(P.counter, 1);
      } else {
        const int j = atomicAdd(P.counter2, 1);
        it = j < *P.fail_count ? P.fail_items[j] : P.n_items;
      }
      item_sh = it;
    }
    __syncthreads();
    const int item = item_sh;
    __syncthreads();
    if (item >= P.n_items) break;
    const int seg = item % P.S;
    const int r = item / P.S;
    const int qb = P.nqb - 1 - (r % P.nqb);
    const int b = r / P.nqb;
    const int t0 = qb * TQ;
    const int t_end = min(a.Lq, t0 + TQ);
    const int p_max = a.Lk - a.Lq + t_end - 1;
    const int s_lo = seg * P.seg_len;
    const int s_hi = min(min(a.Lk, s_lo + P.seg_len), p_max + 1);
    const int n_tiles = s_hi > s_lo ? (s_hi - s_lo + kTileKeys - 1) / kTileKeys : 0;

    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k) + (size_t)b * a.Lk * RB;
    const float* kscale = fp8 ? a.k_scale + (size_t)b * a.Lk : nullptr;
    // key tile [s0, s0 + 64) into ktile[buf] by direct-to-LDS loads (rows past Lk read
    // the last key; they are never admitted)
    auto issue_tile = [&](int s0, int buf) {
#pragma unroll
      for (int u = 0; u < kDmaPerWave; ++u) {
        const int j = wv_id + 4 * u;
        const int piece = j * 64 + lane;
        const int row = piece / kChunks;
        const int cs = piece - row * kChunks;
        const int key = min(s0 + row, a.Lk - 1);
        dma_16(kbase + (size_t)key * RB + 16 * tile_chunk<DT>(row, cs), lds_offset(&ktile[buf][j * 1024]));
      }
      if (fp8 && wv_id == 0) dma_4(kscale + min(s0 + lane, a.Lk - 1), lds_offset(&kscl[buf][0]));
    };
    const int tile_loads = kDmaPerWave + ((fp8 && wv_id == 0) ? 1 : 0);   // per issue_tile, this wave

    // query operands of this wave's tokens (rows past Lq reuse row t0; never appended)
    Op<DT> A[TW][HB];
    int p_t[TW];
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      const int t = t0 + wv_id * TW + tt;
      const int tc = t < a.Lq ? t : t0;
      p_t[tt] = t < a.Lq ? a.Lk - a.Lq + t : -1;
      const uint8_t* qptr = reinterpret_cast<const uint8_t*>(a.q) + ((size_t)b * a.Lq + tc) * H_I * RB;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) A[tt][hb] = load_op<DT>(qptr + (size_t)(hb * 16 + (lane & 15)) * RB, g);
    }
    for (int e = threadIdx.x; e < TQ * H_I; e += 256) {
      const int tt = e / H_I, j = e - tt * H_I;
      const int t = t0 + tt;
      float v = 0.f;
      if (t < a.Lq) {
        v = a.w[((size_t)b * a.Lq + t) * H_I + j];
        if (fp8) v *= a.q_scale[(size_t)b * a.Lq + t];
      }
      wsh[e] = v;
    }
    // complete these loads here, not inside the tile loop where the counter also
    // covers the in-flight tile loads
    __builtin_amdgcn_s_waitcnt(0);

    // the head weights of this wave's tokens stay in registers for the whole item
    __syncthreads();  // wsh filled by the whole workgroup
    f32x4 W[TW][HB];
#pragma unroll
    for (int tt = 0; tt < TW; ++tt)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
        W[tt][hb] = *reinterpret_cast<const f32x4*>(&wsh[(wv_id * TW + tt) * H_I + hb * 16 + 4 * g]);

    uint32_t theta[TW], cnt[TW], scnt[TW];
    float theta_f[TW];  // the float whose order key is theta (-inf: admit every key)
    uint32_t* rk[TW];
    uint32_t* rp[TW];
    bool spec[TW];
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      spec[tt] = false;
      theta[tt] = 0u;
      theta_f[tt] = -INFINITY;
      scnt[tt] = 0u;
      cnt[tt] = 0u;
      rk[tt] = P.row_keys + ((size_t)blockIdx.x * TQ + wv_id * TW + tt) * P.cap;
      rp[tt] = P.row_pos + ((size_t)blockIdx.x * TQ + wv_id * TW + tt) * P.cap;
    }

    // Sample pass (speculative pass only): tiles at s_lo + j * step, all causal for every
    // token of the item; the order keys of this wave's tokens go to its histogram area
    // (TW * 64 * kSampleTiles entries), in the same tile ring as the main pass.
    const int samp_hi = min(s_hi, a.Lk - a.Lq + t0 + 1);
    if (P.pass == 0 && samp_hi - s_lo >= kSampleMinSpan) {   // workgroup-uniform
      const int step = (samp_hi - s_lo - kTileKeys) / (kSampleTiles - 1);
      uint32_t* skeys = hist[wv_id];
#pragma unroll
      for (int u = 0; u < kBufs - 1; ++u) issue_tile(s_lo + u * step, u);
      int cb = 0;
      for (int j = 0; j < kSampleTiles; ++j) {
        if (kBufs == 3 && j + 1 < kSampleTiles) wait_vm_at_most<kDmaPerWave + 1>(tile_loads);
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const int nb = cb == 0 ? kBufs - 1 : cb - 1;
        if (j + kBufs - 1 < kSampleTiles) issue_tile(s_lo + (j + kBufs - 1) * step, nb);
        Op<DT> Bk[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) Bk[kb] = load_op_tile<DT>(ktile[cb], kb * 16 + (lane & 15), g);
        const float ks = fp8 ? kscl[cb][lane] : 1.f;
        float sc[TW];
        tile_scores<DT, HB, TW>(A, Bk, W, sc);
#pragma unroll
        for (int tt = 0; tt < TW; ++tt) skeys[(tt * kSampleTiles + j) * 64 + lane] = order_key(sc[tt] * ks);
        cb = cb + 1 == kBufs ? 0 : cb + 1;
      }
      __syncthreads();   // every wave is done with the ring before the main pass refills it
      wave_lds_fence();
#pragma unroll
      for (int tt = 0; tt < TW; ++tt) {
        const int n = p_t[tt] + 1;   // the token's causal keys (all segments)
        if (n < kSpecMinKeys) continue;
        const float mu = (float)(64 * kSampleTiles) * (float)P.k / (float)n;
        // margin: 4 standard deviations, 6 when the merge takes the largest of a row's
        // segment thresholds (a failing row costs a second pass as long as one item)
        const int jj = (int)ceilf(mu + (P.S > 1 ? 6.f : 4.f) * sqrtf(mu) + 1.f);
        if (jj > 64 * kSampleTiles) continue;
        uint32_t v[kSampleTiles];
#pragma unroll
        for (int q = 0; q < kSampleTiles; ++q) v[q] = skeys[(tt * kSampleTiles + q) * 64 + lane];
        // the largest 16-bit key prefix with at least jj sample keys at or above it is at
        // most the jj-th largest sample key
        uint32_t pre = 0u;
        for (int bit = 31; bit >= 16; --bit) {
          const uint32_t cand = pre | (1u << bit);
          int c = 0;
#pragma unroll
          for (int q = 0; q < kSampleTiles; ++q) c += popc64(ballot(v[q] >= cand));
          if (c >= jj) pre = cand;
        }
        // a positive finite threshold only (then val > theta_f is key > theta)
        if (pre > 0x80000000u && pre < 0xFF800000u) {
          spec[tt] = true;
          theta[tt] = pre;
          theta_f[tt] = key_to_float(pre);
        }
      }
      wave_lds_fence();   // the histogram area is reused by the list selections
    }
    uint32_t theta0[TW];   // starting thresholds (recorded for the merge when S > 1)
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) theta0[tt] = theta[tt];

#pragma unroll
    for (int u = 0; u < kBufs - 1; ++u)
      if (u < n_tiles) issue_tile(s_lo + u * kTileKeys, u);
    int cur = 0;   // it % kBufs
    for (int it = 0; it < n_tiles; ++it) {
      const int s0 = s_lo + it * kTileKeys;
      // this tile has landed (the loads of the later tiles already issued may be pending)
      if (kBufs == 3 && it + 1 < n_tiles) wait_vm_at_most<kDmaPerWave + 1>(tile_loads);
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();   // ... for every wave; the buffer of tile it - 1 is free
      // Issue priority among the waves sharing a SIMD (two workgroups per CU): a wave's
      // admission step (ballots, staging writes, list flushes), which ends at the next
      // tile barrier that the other waves of its workgroup wait on, goes before another
      // wave's scoring (2 over 1), and the scoring before the row loads of the next tile
      // (0).  Timed at 128K: 2% faster than equal priorities, identical index sets.
      __builtin_amdgcn_s_setprio(0);
      const int nxt = cur == 0 ? kBufs - 1 : cur - 1;   // (it + kBufs - 1) % kBufs
      if (it + kBufs - 1 < n_tiles) issue_tile(s0 + (kBufs - 1) * kTileKeys, nxt);

      __builtin_amdgcn_s_setprio(1);
      Op<DT> Bk[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) Bk[kb] = load_op_tile<DT>(ktile[cur], kb * 16 + (lane & 15), g);
      const float ks = fp8 ? kscl[cur][lane] : 1.f;
      const int s = s0 + lane;

      int p_last = p_t[0], p_first = p_t[0];   // the wave's largest / smallest causal end
#pragma unroll
      for (int tt = 1; tt < TW; ++tt) {
        p_last = max(p_last, p_t[tt]);
        p_first = min(p_first, p_t[tt]);
      }
      if (p_last < s0) {   // wave-uniform: every token past its causal range / absent
        cur = cur + 1 == kBufs ? 0 : cur + 1;
        continue;
      }
      float sc[TW];
      tile_scores<DT, HB, TW>(A, Bk, W, sc);
      __builtin_amdgcn_s_setprio(2);
      // Admission: val > theta_f is key > theta (the order-key map is strictly increasing
      // on floats with -0 = +0).  Positions are checked only in a tile that crosses a
      // token's causal edge or the segment end (a separate copy of the loop body, so the
      // other tiles carry no masking).
      auto admit = [&](auto edge_tag) {
        constexpr bool kEdge = decltype(edge_tag)::value;
#pragma unroll
        for (int tt = 0; tt < TW; ++tt) {
          if (p_t[tt] < s0) continue;  // wave-uniform: token past its causal range / absent
          const float val = sc[tt] * ks;
          bool pred = val > theta_f[tt];
          if constexpr (kEdge) pred = pred && (s <= p_t[tt]) && (s < s_hi);
          const uint64_t m = ballot(pred);
          if (m) {
            if (pred) stg[wv_id * TW + tt][scnt[tt] + rank_below(m)] = make_uint2(__float_as_uint(val), (uint32_t)s);
            scnt[tt] += popc64(m);
          }
        }
      };
      if (s0 + kTileKeys - 1 > p_first || s0 + kTileKeys > s_hi) admit(std::true_type{});
      else admit(std::false_type{});
#pragma unroll
      for (int tt = 0; tt < TW; ++tt) {
        if (scnt[tt] > (uint32_t)(kStage - kTileKeys)) {
          cnt[tt] = flush_stage(stg[wv_id * TW + tt], scnt[tt], rk[tt], rp[tt], cnt[tt]);
          scnt[tt] = 0;
          if (cnt[tt] > (uint32_t)(P.cap - kStage)) {
            cnt[tt] = shrink_list(rk[tt], rp[tt], cnt[tt], (uint32_t)P.k, (uint32_t)(P.cap + P.k) / 2,
                                  hist[wv_id], theta[tt]);
            theta_f[tt] = key_to_float(theta[tt]);
          }
        }
      }
      cur = cur + 1 == kBufs ? 0 : cur + 1;
    }

    __builtin_amdgcn_s_setprio(0);
    // finalize this wave's rows
#pragma unroll
    for (int tt = 0; tt < TW; ++tt)
      cnt[tt] = flush_stage(stg[wv_id * TW + tt], scnt[tt], rk[tt], rp[tt], cnt[tt]);
    __threadfence_block();
    // one call per token of the wave (unrolled by hand: the selection is large)
    auto finish_row = [&](const int tt) {
      const int t = t0 + wv_id * TW + tt;
      if (t >= a.Lq) return;
      const int n_causal = max(0, min(p_t[tt] + 1, s_hi) - s_lo);
      if (P.S == 1 && spec[tt] && cnt[tt] < (uint32_t)min(P.k, n_causal)) {
        // too few keys passed the speculative threshold: the item is recomputed exactly
        if (lane == 0) P.fail_items[atomicAdd(P.fail_count, 1)] = item;
      }
      const size_t row = (size_t)b * a.Lq + t;
      // the top k go straight to the row's index row (one key segment: positions, -1 past
      // a short list) or to the segment's list (keys and positions)
      const bool one = P.S == 1;
      int32_t* out = P.idx + row * P.k;
      uint32_t* ok = P.seg_keys + row * P.seg_stride + (size_t)seg * P.k;
      uint32_t* op = P.seg_pos + row * P.seg_stride + (size_t)seg * P.k;
      cnt[tt] = select_to(rk[tt], rp[tt], cnt[tt], (uint32_t)P.k, hist[wv_id],
                          [=](uint32_t d, uint32_t key, uint32_t p) {
                            if (one) {
                              out[d] = (int32_t)p;
                            } else {
                              ok[d] = key;
                              op[d] = p;
                            }
                          });
      if (one) {
        for (int j = (int)cnt[tt] + lane; j < P.k; j += 64) out[j] = -1;
      } else {
        if (lane == 0) {
          P.seg_cnt[row * P.S + seg] = (int32_t)cnt[tt];
          P.seg_spec[row * P.S + seg] = spec[tt] ? theta0[tt] : 0u;
        }
      }
    };
    finish_row(0);
    if constexpr (TW > 1) finish_row(1);
    static_assert(TW <= 2, "finish_row calls");
  }
}

// Merge of per-segment top-k lists (segments are in position order, so their
// concatenation is in ascending position order).  One wave per query row.
// Speculation check of the merge (mode 1, after the first fused launch): a row whose
// segment lists hold fewer than min(k, its causal keys) entries is flagged, and every
// segment item of its query block is recorded for the second fused launch; mode 2 (after
// it) merges only the flagged rows.
struct MergeSpec {
  int mode;             // 1: check and record failures; 2: flagged rows only
  int Lq, Lk, nqb, TQ;
  const uint32_t* seg_spec;
  int* fail_count;
  int* fail_items;
  int* row_flag;        // [rows], zeroed before mode 1
};

__global__ __launch_bounds__(256) void merge_segments_kernel(uint32_t* seg_keys, uint32_t* seg_pos,
                                                             const int32_t* seg_cnt, int rows, int S, int k, int stride,
                                                             int32_t* idx, MergeSpec M) {
  __shared__ uint32_t hist[4][kBins];
  const int lane = threadIdx.x & 63, wv_id = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wv_id;
  if (row >= rows) return;
  if (M.mode == 2 && M.row_flag[row] == 0) return;
  uint32_t theta_max = 0;   // largest starting threshold among the row's segments
  if (M.mode == 1)
    for (int sg = 0; sg < S; ++sg) theta_max = max(theta_max, M.seg_spec[(size_t)row * S + sg]);
  uint32_t* bk = seg_keys + (size_t)row * stride;
  uint32_t* bp = seg_pos + (size_t)row * stride;
  // pack the lists contiguously at the start of the row's region (moves only downwards),
  // counting the entries above theta_max
  uint32_t n = 0, above = 0;
  for (int sg = 0; sg < S; ++sg) {
    const uint32_t c = (uint32_t)seg_cnt[(size_t)row * S + sg];
    for (uint32_t j0 = 0; j0 < c; j0 += 64) {
      const uint32_t j = j0 + lane;
      uint32_t kk = 0, pp = 0;
      if (j < c) {
        kk = bk[(size_t)sg * k + j];
        pp = bp[(size_t)sg * k + j];
      }
      if (j < c) {
        bk[n + j] = kk;
        bp[n + j] = pp;
      }
      above += (uint32_t)popc64(ballot(j < c && kk > theta_max));
    }
    n += c;
  }
  if (M.mode == 1 && theta_max != 0u) {
    const int n_causal = M.Lk - M.Lq + (row % M.Lq) + 1;
    if (above < (uint32_t)min(k, n_causal)) {
      // a top-k key may lie below some segment's threshold: recompute the row's block
      if (lane == 0) {
        M.row_flag[row] = 1;
        const int b = row / M.Lq, qb = (row % M.Lq) / M.TQ;
        const int r = b * M.nqb + (M.nqb - 1 - qb);
        for (int sg = 0; sg < S; ++sg) M.fail_items[atomicAdd(M.fail_count, 1)] = r * S + sg;
      }
      return;
    }
  }
  uint32_t kth;
  n = reduce_to_k(bk, bp, n, (uint32_t)k, hist[wv_id], kth);
  int32_t* out = idx + (size_t)row * k;
  for (int j = lane; j < k; j += 64) out[j] = j < (int)n ? (int32_t)bp[j] : -1;
}

__global__ void zero_ints_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
template <int DT>
static hipError_t rowscan_dispatch(const IndexerArgs& a, float* scores, int64_t stride, uint32_t* row_hist,
                                   hipStream_t s) {
  const int chunk = rowscan_chunk(a.B * a.Lq, a.Lk);
  dim3 grid((unsigned)((a.Lk + chunk - 1) / chunk) * (unsigned)(a.B * a.Lq));
  switch (a.H_I / 16) {
    case 1: indexer_rowscan_kernel<DT, 1><<<grid, 256, 0, s>>>(a, scores, stride, row_hist, chunk); break;
    case 2: indexer_rowscan_kernel<DT, 2><<<grid, 256, 0, s>>>(a, scores, stride, row_hist, chunk); break;
    case 3: indexer_rowscan_kernel<DT, 3><<<grid, 256, 0, s>>>(a, scores, stride, row_hist, chunk); break;
    default: indexer_rowscan_kernel<DT, 4><<<grid, 256, 0, s>>>(a, scores, stride, row_hist, chunk); break;
  }
  return hipGetLastError();
}

__global__ void zero_words_kernel(uint32_t* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  zero_words_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_indexer_scores(const IndexerArgs& a, float* scores, int64_t stride, uint32_t* row_hist,
                                 hipStream_t s) {
  if (a.dtype == DSA_F32) {
    dim3 grid((unsigned)((a.Lk + 255) / 256) * (unsigned)(a.B * a.Lq));
    const size_t smem = (size_t)(a.H_I * a.d_I + a.H_I) * sizeof(float);
    indexer_f32_kernel<<<grid, 256, smem, s>>>(a, scores, stride, row_hist);
    return hipGetLastError();
  }
  if (a.dtype == DSA_BF16) return rowscan_dispatch<DSA_BF16>(a, scores, stride, row_hist, s);
  return rowscan_dispatch<DSA_FP8_E4M3>(a, scores, stride, row_hist, s);
}

static ChunkLists plan_lists(int rows, int Lk) {
  ChunkLists L{};
  L.chunk = min(rowscan_chunk(rows, Lk), kSelMaxChunk);
  L.n_chunks = (Lk + L.chunk - 1) / L.chunk;
  L.row_stride = ((int64_t)Lk + 63) / 64 * 64 + kSelMaxChunk;
  return L;
}

// Device-independent bound: n_chunks * chunk < Lk + kSelMaxChunk <= row_stride, and a
// chunk has at least 64 keys.
size_t chunk_lists_ws(int rows, int Lk) {
  const size_t stride = ((size_t)Lk + 63) / 64 * 64 + kSelMaxChunk;
  const size_t lists = ((size_t)rows * stride * 2 * sizeof(uint32_t) + 255) / 256 * 256;
  const size_t cnt = ((size_t)rows * ((Lk + 63) / 64) * sizeof(uint32_t) + 255) / 256 * 256;
  const size_t hist = (size_t)rows * kRowHistBins * sizeof(uint32_t);
  return lists + cnt + hist;
}

template <int DT>
static void chunksel_dispatch(const IndexerArgs& a, int k, const ChunkLists& L, int rows, hipStream_t s) {
  const dim3 grid((unsigned)(rows * L.n_chunks));
  switch (a.H_I / 16) {
    case 1: indexer_chunksel_kernel<DT, 1><<<grid, 256, 0, s>>>(a, k, L); break;
    case 2: indexer_chunksel_kernel<DT, 2><<<grid, 256, 0, s>>>(a, k, L); break;
    case 3: indexer_chunksel_kernel<DT, 3><<<grid, 256, 0, s>>>(a, k, L); break;
    default: indexer_chunksel_kernel<DT, 4><<<grid, 256, 0, s>>>(a, k, L); break;
  }
}

hipError_t launch_indexer_topk_lists(const IndexerArgs& a, int k, const int32_t* seq_lens, const PagedCache& pc,
                                     int32_t* idx, void* ws, size_t ws_bytes, hipStream_t s) {
  const int rows = a.B * a.Lq;
  if (ws_bytes < chunk_lists_ws(rows, a.Lk)) return hipErrorInvalidValue;
  ChunkLists L = plan_lists(rows, a.Lk);
  L.seq_lens = seq_lens;
  L.block_table = pc.block_table;
  L.max_pages = pc.max_pages;
  L.page_log2 = pc.block_table ? pc.page_log2 : 0;
  L.pool_pages = pc.pool_pages;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  const size_t lists = ((size_t)rows * L.row_stride * 2 * sizeof(uint32_t) + 255) / 256 * 256;
  const size_t cnt = ((size_t)rows * ((a.Lk + 63) / 64) * sizeof(uint32_t) + 255) / 256 * 256;
  L.keys = reinterpret_cast<uint32_t*>(w8);
  L.pos = L.keys + (size_t)rows * L.row_stride;
  L.cnt = reinterpret_cast<uint32_t*>(w8 + lists);
  L.row_hist = reinterpret_cast<uint32_t*>(w8 + lists + cnt);
  hipError_t e = launch_zero(L.row_hist, (size_t)rows * kRowHistBins * sizeof(uint32_t), s);
  if (e != hipSuccess) return e;
  if (a.dtype == DSA_BF16) chunksel_dispatch<DSA_BF16>(a, k, L, rows, s);
  else chunksel_dispatch<DSA_FP8_E4M3>(a, k, L, rows, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  lists_filter_kernel<<<dim3(L.n_chunks, rows), 256, 0, s>>>(L, a.Lq, a.Lk, k);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_lists_finish(L, rows, a.Lq, a.Lk, k, idx, s);
}

__global__ __launch_bounds__(256) void paged_rows_kernel(const int32_t* __restrict__ idx, int64_t n, int Lq, int k,
                                                         PagedCache pc, int32_t* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const int b = (int)(e / ((int64_t)Lq * k));
  const int v = idx[e];
  const int lp = v >> pc.page_log2;
  int r = -1;
  if (v >= 0 && lp < pc.max_pages) {
    const int pg = pc.block_table[(size_t)b * pc.max_pages + lp];
    if (pg >= 0 && pg < pc.pool_pages) r = (pg << pc.page_log2) | (v & ((1 << pc.page_log2) - 1));
  }
  out[e] = r;
}

hipError_t launch_paged_rows(const int32_t* idx, int B, int Lq, int k, const PagedCache& pc, int32_t* rows_out,
                             hipStream_t s) {
  const int64_t n = (int64_t)B * Lq * k;
  if (n == 0) return hipSuccess;
  paged_rows_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(idx, n, Lq, k, pc, rows_out);
  return hipGetLastError();
}

struct FusedPlan {
  int TQ, nqb, S, seg_len, n_items, grid, cap, seg_stride;
  size_t off_rowbuf, off_seg, off_cnt, off_fail, off_flag, total;
};

static FusedPlan plan_fused(int B, int Lq, int Lk, int k, int dtype) {
  FusedPlan p;
  p.TQ = 4 * (dtype == DSA_FP8_E4M3 ? IdxTraits<DSA_FP8_E4M3>::kTokensPerWave
                                     : IdxTraits<DSA_BF16>::kTokensPerWave);
  p.nqb = (Lq + p.TQ - 1) / p.TQ;
  const long long base_items = (long long)B * p.nqb;
  // Split the keys when there are too few query blocks to fill the GPU (chunked
  // prefill); each segment keeps at least 8192 keys.
  int S = 1;
  if (base_items < 2048) {
    S = (int)((2048 + base_items - 1) / base_items);
    const int max_s = (Lk + 8191) / 8192;
    if (S > max_s) S = max_s;
    if (S < 1) S = 1;
  }
  p.S = S;
  p.seg_len = ((Lk + S - 1) / S + kTileKeys - 1) / kTileKeys * kTileKeys;
  p.n_items = (int)(base_items * S);
  p.grid = p.n_items < kPersistentGrid ? p.n_items : kPersistentGrid;
  p.cap = topk_buffer_capacity(k);
  size_t off = 256;  // work counter
  p.off_rowbuf = off;
  off += (size_t)p.grid * p.TQ * p.cap * sizeof(uint32_t) * 2;
  off = (off + 255) / 256 * 256;
  p.off_seg = off;
  p.seg_stride = (S * k + 3) / 4 * 4;  // 16-byte aligned rows
  if (S > 1) off += (size_t)B * Lq * p.seg_stride * sizeof(uint32_t) * 2;
  off = (off + 255) / 256 * 256;
  p.off_cnt = off;
  if (S > 1) off += (size_t)B * Lq * S * sizeof(int32_t) * 2;   // counts, then starting thresholds
  off = (off + 255) / 256 * 256;
  p.off_fail = off;                  // failed items of the speculative pass, then row flags
  off += (size_t)p.n_items * 8 * sizeof(int32_t);
  off = (off + 255) / 256 * 256;
  p.off_flag = off;
  if (S > 1) off += (size_t)B * Lq * sizeof(int32_t);
  p.total = (off + 255) / 256 * 256;
  return p;
}

size_t indexer_topk_fused_ws(int B, int Lq, int Lk, int k, int dtype) {
  return plan_fused(B, Lq, Lk, k, dtype).total;
}

template <int DT>
static void fused_dispatch(const FusedParams& P, int grid, int HB, hipStream_t s) {
  switch (HB) {
    case 1: indexer_topk_kernel<DT, 1><<<grid, 256, 0, s>>>(P); break;
    case 2: indexer_topk_kernel<DT, 2><<<grid, 256, 0, s>>>(P); break;
    case 3: indexer_topk_kernel<DT, 3><<<grid, 256, 0, s>>>(P); break;
    default: indexer_topk_kernel<DT, 4><<<grid, 256, 0, s>>>(P); break;
  }
}

hipError_t launch_indexer_topk_fused(const IndexerArgs& a, int k, int32_t* idx, void* ws,
                                     size_t ws_bytes, hipStream_t s) {
  const FusedPlan pl = plan_fused(a.B, a.Lq, a.Lk, k, a.dtype);
  if (ws_bytes < pl.total) return hipErrorInvalidValue;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  FusedParams P;
  P.a = a;
  P.k = k;
  P.cap = pl.cap;
  P.S = pl.S;
  P.seg_len = pl.seg_len;
  P.nqb = pl.nqb;
  P.n_items = pl.n_items;
  P.idx = idx;
  P.row_keys = reinterpret_cast<uint32_t*>(w8 + pl.off_rowbuf);
  P.row_pos = P.row_keys + (size_t)pl.grid * pl.TQ * pl.cap;
  P.seg_keys = reinterpret_cast<uint32_t*>(w8 + pl.off_seg);
  P.seg_stride = pl.seg_stride;
  P.seg_pos = P.seg_keys + (size_t)a.B * a.Lq * pl.seg_stride;
  P.seg_cnt = reinterpret_cast<int32_t*>(w8 + pl.off_cnt);
  // [0] work counter, [1] pass-1 counter, [2] failures, [8..15] per-XCD work counters (S > 1)
  P.counter = reinterpret_cast<int*>(w8);
  P.counter2 = P.counter + 1;
  P.fail_count = P.counter + 2;
  P.fail_items = reinterpret_cast<int*>(w8 + pl.off_fail);
  P.pass = 0;
  const int rows = a.B * a.Lq;
  P.seg_spec = reinterpret_cast<uint32_t*>(P.seg_cnt + (size_t)a.B * a.Lq * pl.S);
  MergeSpec M{1, a.Lq, a.Lk, pl.nqb, pl.TQ, P.seg_spec, P.fail_count, P.fail_items,
              reinterpret_cast<int*>(w8 + pl.off_flag)};
  zero_ints_kernel<<<1, 64, 0, s>>>(P.counter, 16);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && pl.S > 1) e = launch_zero(M.row_flag, (size_t)rows * sizeof(int32_t), s);
  if (e != hipSuccess) return e;
  auto fused = [&]() {
    if (a.dtype == DSA_BF16) fused_dispatch<DSA_BF16>(P, pl.grid, a.H_I / 16, s);
    else fused_dispatch<DSA_FP8_E4M3>(P, pl.grid, a.H_I / 16, s);
    return hipGetLastError();
  };
  auto merge = [&](int mode) {
    M.mode = mode;
    merge_segments_kernel<<<(rows + 3) / 4, 256, 0, s>>>(P.seg_keys, P.seg_pos, P.seg_cnt, rows, pl.S, k,
                                                         pl.seg_stride, idx, M);
    return hipGetLastError();
  };
  // pass 0 (speculative thresholds), the merge's check when the keys are segmented, pass 1
  // over the recorded items (exact), and the merge of the rows it recomputed
  e = fused();
  if (e == hipSuccess && pl.S > 1) e = merge(1);
  P.pass = 1;
  if (e == hipSuccess) e = fused();
  if (e == hipSuccess && pl.S > 1) e = merge(2);
  return e;
}

}  // namespace dsa
