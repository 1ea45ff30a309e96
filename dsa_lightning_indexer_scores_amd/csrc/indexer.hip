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
#include "dsa_common.hpp"
#include "dsa_launch.hpp"
#include "../../include/dsa.h"

namespace dsa {

constexpr int kTileKeys = 64;
constexpr int kPersistentGrid = 1024;  // fixed so that workspace sizes are pure host math

template <int DT> struct IdxTraits;
template <> struct IdxTraits<DSA_BF16> {
  static constexpr int kRowBytes = 256;   // d_I = 128 bf16
  static constexpr int kLdsStride = 272;  // +16 B: 16 consecutive rows hit distinct banks
  static constexpr int kTokensPerWave = 2;
};
template <> struct IdxTraits<DSA_FP8_E4M3> {
  static constexpr int kRowBytes = 128;   // d_I = 128 E4M3
  static constexpr int kLdsStride = 144;
  static constexpr int kTokensPerWave = 4;
};

// Per-lane operand slice of one 16-row block of a d_I = 128 row: lane group g = lane/16
// takes bytes [g * kRowBytes/4, (g+1) * kRowBytes/4).  A (queries) and B (keys) use the
// same slice, so the MFMA pairs equal feature indices.
template <int DT> struct Op;
template <> struct Op<DSA_FP8_E4M3> { i32x8 v; };
template <> struct Op<DSA_BF16> { bf16x8 v[4]; };

template <int DT>
__device__ __forceinline__ Op<DT> load_op(const uint8_t* row, int g);
template <>
__device__ __forceinline__ Op<DSA_FP8_E4M3> load_op<DSA_FP8_E4M3>(const uint8_t* row, int g) {
  const i32x4* p = reinterpret_cast<const i32x4*>(row + 32 * g);
  i32x4 lo = p[0], hi = p[1];
  Op<DSA_FP8_E4M3> o;
  o.v = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return o;
}
template <>
__device__ __forceinline__ Op<DSA_BF16> load_op<DSA_BF16>(const uint8_t* row, int g) {
  const bf16x8* p = reinterpret_cast<const bf16x8*>(row + 64 * g);
  Op<DSA_BF16> o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o.v[i] = p[i];
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

// Scores of one token against a 64-key tile.  a[hb]: the token's heads 16hb..16hb+15;
// b[kb]: keys 16kb..16kb+15 of the tile; wv[hb][i] = w'[16hb + 4g + i].
// Returns, in lane l, sum_j w'_j ReLU(q_j . k_{s0+l}) (before the fp8 key scale).
// Shared by the materialising and the fused kernels so both produce identical bits.
template <int DT, int HB>
__device__ __forceinline__ float tile_score(const Op<DT> (&a)[HB], const Op<DT> (&b)[4],
                                            const f32x4 (&wv)[HB]) {
  float p[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    float acc = 0.f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const f32x4 d = dot16<DT>(a[hb], b[kb]);
      acc = fmaf(wv[hb][0], fmaxf(d[0], 0.f), acc);
      acc = fmaf(wv[hb][1], fmaxf(d[1], 0.f), acc);
      acc = fmaf(wv[hb][2], fmaxf(d[2], 0.f), acc);
      acc = fmaf(wv[hb][3], fmaxf(d[3], 0.f), acc);
    }
    p[kb] = acc;
  }
  return reduce_scatter4(p[0], p[1], p[2], p[3]);
}

// ---------------------------------------------------------------------------
// Materialised scores: one workgroup per (query row, chunk of keys); each wave scans
// every fourth 64-key tile of the chunk, reading k^I straight from HBM (no reuse).
// ---------------------------------------------------------------------------
constexpr int kRowscanChunk = 4096;

template <int DT, int HB>
__global__ __launch_bounds__(256) void indexer_rowscan_kernel(IndexerArgs a, float* __restrict__ scores) {
  constexpr int RB = IdxTraits<DT>::kRowBytes;
  const int n_chunks = (a.Lk + kRowscanChunk - 1) / kRowscanChunk;
  const int qrow = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x - qrow * n_chunks;
  const int b = qrow / a.Lq, i = qrow - b * a.Lq;
  const int p = a.Lk - a.Lq + i;
  const int lane = threadIdx.x & 63, wv_id = threadIdx.x >> 6, g = lane >> 4;
  const int s_begin = chunk * kRowscanChunk;
  const int s_end = min(a.Lk, s_begin + kRowscanChunk);
  float* out = scores + (size_t)qrow * a.Lk;

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
  for (int s0 = s_begin + wv_id * kTileKeys; s0 < s_end; s0 += 4 * kTileKeys) {
    const int s = s0 + lane;
    if (s0 > p) {  // whole tile is non-causal for this query
      if (s < s_end) out[s] = -INFINITY;
      continue;
    }
    Op<DT> Bk[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = min(s0 + kb * 16 + (lane & 15), a.Lk - 1);
      Bk[kb] = load_op<DT>(kbase + (size_t)key * RB, g);
    }
    float val = tile_score<DT, HB>(A, Bk, W);
    if (DT == DSA_FP8_E4M3) val *= ksc[min(s, a.Lk - 1)];
    if (s < s_end) out[s] = (s <= p) ? val : -INFINITY;
  }
}

// Reference-size fp32 path: one thread per (query, key); q row and weights in LDS.
__global__ __launch_bounds__(256) void indexer_f32_kernel(IndexerArgs a, float* __restrict__ scores) {
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
  }
  scores[(size_t)qrow * a.Lk + s] = val;
}

// ---------------------------------------------------------------------------
// Wave-level exact selection on a candidate array (global memory, ascending positions).
// ---------------------------------------------------------------------------

// Radix-select the k-th largest order key among buf[0..n) (n > k), 8 bits per pass.
// Returns theta (the k-th key) and need_eq (how many entries equal to theta belong to
// the top k: the first need_eq of them in array order).
__device__ void wave_select(const uint2* buf, uint32_t n, uint32_t k, uint32_t* hist,
                            uint32_t& theta, uint32_t& need_eq) {
  const int lane = lane_id();
  uint32_t prefix = 0, pmask = 0, krem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) hist[4 * lane + j] = 0;
    wave_lds_fence();
    for (uint32_t e = lane; e < n; e += 64) {
      const uint32_t key = buf[e].x;
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    wave_lds_fence();
    const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                   h3 = hist[4 * lane + 3];
    const uint32_t tot = h0 + h1 + h2 + h3;
    uint32_t S = tot;  // inclusive suffix sum over lanes >= this lane
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = __shfl_down(S, d);
      if (lane + d < 64) S += o;
    }
    const uint32_t above = S - tot;  // entries whose digit lies in higher lanes' bins
    const bool here = (above < krem) && (S >= krem);
    const uint64_t m = ballot(here);
    const int src = __ffsll((long long)m) - 1;
    uint32_t c = above, d;
    if (c + h3 >= krem) d = 4 * lane + 3;
    else { c += h3;
      if (c + h2 >= krem) d = 4 * lane + 2;
      else { c += h2;
        if (c + h1 >= krem) d = 4 * lane + 1;
        else { c += h1; d = 4 * lane; } } }
    d = __shfl(d, src);
    c = __shfl(c, src);
    prefix |= d << shift;
    pmask |= 255u << shift;
    krem -= c;
    wave_lds_fence();
  }
  theta = prefix;
  need_eq = krem;
}

// In-place stable compaction keeping keys > theta and the first need_eq keys == theta.
__device__ uint32_t wave_compact(uint2* buf, uint32_t n, uint32_t theta, uint32_t need_eq) {
  const int lane = lane_id();
  uint32_t out = 0, eq_seen = 0;
  for (uint32_t base = 0; base < n; base += 64) {
    const uint32_t e = base + lane;
    const bool v = e < n;
    const uint2 x = v ? buf[e] : make_uint2(0u, 0u);
    const bool gt = v && x.x > theta;
    const bool eq = v && x.x == theta;
    const uint64_t meq = ballot(eq);
    const bool take = gt || (eq && eq_seen + rank_below(meq) < need_eq);
    const uint64_t mt = ballot(take);
    if (take) buf[out + rank_below(mt)] = x;  // destination <= e: never ahead of reads
    out += popc64(mt);
    eq_seen += popc64(meq);
  }
  return out;
}

// ---------------------------------------------------------------------------
// Fused streaming indexer + top-k (persistent workgroups, atomic work queue).
// Work item = (sequence, block of TQ consecutive queries, key segment); blocks with the
// most causal keys are dispatched first.  With one segment the kernel writes idx
// directly; with several it writes each segment's top-k list for a merge kernel.
// ---------------------------------------------------------------------------
struct FusedParams {
  IndexerArgs a;
  int k, cap, S, seg_len, nqb, n_items;
  int32_t* idx;
  uint2* rowbuf;
  uint2* seg_out;
  int32_t* seg_cnt;
  int* counter;
};

template <int DT, int HB>
__global__ __launch_bounds__(256) void indexer_topk_kernel(FusedParams P) {
  constexpr int RB = IdxTraits<DT>::kRowBytes;
  constexpr int LS = IdxTraits<DT>::kLdsStride;
  constexpr int TW = IdxTraits<DT>::kTokensPerWave;
  constexpr int TQ = 4 * TW;
  constexpr int H_I = HB * 16;
  constexpr int kChunks = RB / 16;                 // 16-byte pieces per key row
  constexpr int kPerThread = 64 * kChunks / 256;   // pieces each thread stages per tile
  __shared__ __attribute__((aligned(16))) uint8_t ktile[2][kTileKeys * LS];
  __shared__ float kscl[2][kTileKeys];
  __shared__ __attribute__((aligned(16))) float wsh[TQ * H_I];
  __shared__ uint32_t hist[4][256];
  __shared__ int item_sh;

  const IndexerArgs& a = P.a;
  const int lane = threadIdx.x & 63, wv_id = threadIdx.x >> 6, g = lane >> 4;
  const bool fp8 = (DT == DSA_FP8_E4M3);

  for (;;) {
    if (threadIdx.x == 0) item_sh = atomicAdd(P.counter, 1);
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

    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k) + (size_t)b * a.Lk * RB;
    const float* kscale = fp8 ? a.k_scale + (size_t)b * a.Lk : nullptr;
    auto load_piece = [&](int s0, int piece) -> i32x4 {
      const int key = piece / kChunks, c = piece - key * kChunks;
      const int s = min(s0 + key, a.Lk - 1);
      return *reinterpret_cast<const i32x4*>(kbase + (size_t)s * RB + 16 * c);
    };
    auto store_piece = [&](int buf, int piece, i32x4 v) {
      const int key = piece / kChunks, c = piece - key * kChunks;
      *reinterpret_cast<i32x4*>(&ktile[buf][key * LS + 16 * c]) = v;
    };

    uint32_t theta[TW], cnt[TW];
    uint2* rb[TW];
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      theta[tt] = 0u;
      cnt[tt] = 0u;
      rb[tt] = P.rowbuf + ((size_t)blockIdx.x * TQ + wv_id * TW + tt) * P.cap;
    }

    if (n_tiles > 0) {
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const int piece = threadIdx.x + 256 * j;
        store_piece(0, piece, load_piece(s_lo, piece));
      }
      if (fp8 && threadIdx.x < kTileKeys) kscl[0][threadIdx.x] = kscale[min(s_lo + (int)threadIdx.x, a.Lk - 1)];
    }
    __syncthreads();

    for (int it = 0; it < n_tiles; ++it) {
      const int s0 = s_lo + it * kTileKeys;
      const int cur = it & 1;
      const bool more = it + 1 < n_tiles;
      i32x4 pre[kPerThread];
      float pre_sc = 0.f;
      if (more) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) pre[j] = load_piece(s0 + kTileKeys, threadIdx.x + 256 * j);
        if (fp8 && threadIdx.x < kTileKeys) pre_sc = kscale[min(s0 + kTileKeys + (int)threadIdx.x, a.Lk - 1)];
      }

      Op<DT> Bk[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) Bk[kb] = load_op<DT>(&ktile[cur][(kb * 16 + (lane & 15)) * LS], g);
      const float ks = fp8 ? kscl[cur][lane] : 1.f;
      const int s = s0 + lane;

#pragma unroll
      for (int tt = 0; tt < TW; ++tt) {
        if (p_t[tt] < s0) continue;  // wave-uniform: token past its causal range / absent
        f32x4 W[HB];
        const float* wrow = &wsh[(wv_id * TW + tt) * H_I];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) W[hb] = *reinterpret_cast<const f32x4*>(wrow + hb * 16 + 4 * g);
        const float val = tile_score<DT, HB>(A[tt], Bk, W) * ks;
        const uint32_t key = order_key(val);
        const bool pred = (s <= p_t[tt]) && (s < s_hi) && (key > theta[tt]);
        const uint64_t m = ballot(pred);
        if (m) {
          if (pred) rb[tt][cnt[tt] + rank_below(m)] = make_uint2(key, (uint32_t)s);
          cnt[tt] += popc64(m);
          if (cnt[tt] > (uint32_t)(P.cap - kTileKeys)) {
            __threadfence_block();
            uint32_t th, ne;
            wave_select(rb[tt], cnt[tt], (uint32_t)P.k, hist[wv_id], th, ne);
            cnt[tt] = wave_compact(rb[tt], cnt[tt], th, ne);
            theta[tt] = th;
            __threadfence_block();
          }
        }
      }

      if (more) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) store_piece(cur ^ 1, threadIdx.x + 256 * j, pre[j]);
        if (fp8 && threadIdx.x < kTileKeys) kscl[cur ^ 1][threadIdx.x] = pre_sc;
      }
      __syncthreads();
    }

    // finalize this wave's rows
    __threadfence_block();
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      const int t = t0 + wv_id * TW + tt;
      if (t >= a.Lq) continue;
      if (cnt[tt] > (uint32_t)P.k) {
        uint32_t th, ne;
        wave_select(rb[tt], cnt[tt], (uint32_t)P.k, hist[wv_id], th, ne);
        cnt[tt] = wave_compact(rb[tt], cnt[tt], th, ne);
        __threadfence_block();
      }
      const size_t row = (size_t)b * a.Lq + t;
      if (P.S == 1) {
        int32_t* out = P.idx + row * P.k;
        for (int j = lane; j < P.k; j += 64) out[j] = j < (int)cnt[tt] ? (int32_t)rb[tt][j].y : -1;
      } else {
        uint2* out = P.seg_out + (row * P.S + seg) * P.k;
        for (int j = lane; j < (int)cnt[tt]; j += 64) out[j] = rb[tt][j];
        if (lane == 0) P.seg_cnt[row * P.S + seg] = (int32_t)cnt[tt];
      }
    }
  }
}

// Merge of per-segment top-k lists (segments are in position order, so their
// concatenation is in ascending position order).  One wave per query row.
__global__ __launch_bounds__(256) void merge_segments_kernel(uint2* seg_out, const int32_t* seg_cnt,
                                                             int rows, int S, int k, int32_t* idx) {
  __shared__ uint32_t hist[4][256];
  const int lane = threadIdx.x & 63, wv_id = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wv_id;
  if (row >= rows) return;
  uint2* base = seg_out + (size_t)row * S * k;
  // pack the lists contiguously at the start of the row's region (moves only downwards)
  uint32_t n = 0;
  for (int sg = 0; sg < S; ++sg) {
    const uint32_t c = (uint32_t)seg_cnt[(size_t)row * S + sg];
    const uint2* src = base + (size_t)sg * k;
    for (uint32_t j0 = 0; j0 < c; j0 += 64) {
      const uint32_t j = j0 + lane;
      uint2 v = make_uint2(0u, 0u);
      if (j < c) v = src[j];
      if (j < c) base[n + j] = v;
    }
    n += c;
  }
  __threadfence_block();
  if (n > (uint32_t)k) {
    uint32_t th, ne;
    wave_select(base, n, (uint32_t)k, hist[wv_id], th, ne);
    n = wave_compact(base, n, th, ne);
    __threadfence_block();
  }
  int32_t* out = idx + (size_t)row * k;
  for (int j = lane; j < k; j += 64) out[j] = j < (int)n ? (int32_t)base[j].y : -1;
}

__global__ void zero_ints_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
template <int DT>
static hipError_t rowscan_dispatch(const IndexerArgs& a, float* scores, hipStream_t s) {
  dim3 grid((unsigned)((a.Lk + kRowscanChunk - 1) / kRowscanChunk) * (unsigned)(a.B * a.Lq));
  switch (a.H_I / 16) {
    case 1: indexer_rowscan_kernel<DT, 1><<<grid, 256, 0, s>>>(a, scores); break;
    case 2: indexer_rowscan_kernel<DT, 2><<<grid, 256, 0, s>>>(a, scores); break;
    case 3: indexer_rowscan_kernel<DT, 3><<<grid, 256, 0, s>>>(a, scores); break;
    default: indexer_rowscan_kernel<DT, 4><<<grid, 256, 0, s>>>(a, scores); break;
  }
  return hipGetLastError();
}

hipError_t launch_indexer_scores(const IndexerArgs& a, float* scores, hipStream_t s) {
  if (a.dtype == DSA_F32) {
    dim3 grid((unsigned)((a.Lk + 255) / 256) * (unsigned)(a.B * a.Lq));
    const size_t smem = (size_t)(a.H_I * a.d_I + a.H_I) * sizeof(float);
    indexer_f32_kernel<<<grid, 256, smem, s>>>(a, scores);
    return hipGetLastError();
  }
  if (a.dtype == DSA_BF16) return rowscan_dispatch<DSA_BF16>(a, scores, s);
  return rowscan_dispatch<DSA_FP8_E4M3>(a, scores, s);
}

struct FusedPlan {
  int TQ, nqb, S, seg_len, n_items, grid, cap;
  size_t off_rowbuf, off_seg, off_cnt, total;
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
  off += (size_t)p.grid * p.TQ * p.cap * sizeof(uint2);
  off = (off + 255) / 256 * 256;
  p.off_seg = off;
  if (S > 1) off += (size_t)B * Lq * S * k * sizeof(uint2);
  off = (off + 255) / 256 * 256;
  p.off_cnt = off;
  if (S > 1) off += (size_t)B * Lq * S * sizeof(int32_t);
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
  P.rowbuf = reinterpret_cast<uint2*>(w8 + pl.off_rowbuf);
  P.seg_out = reinterpret_cast<uint2*>(w8 + pl.off_seg);
  P.seg_cnt = reinterpret_cast<int32_t*>(w8 + pl.off_cnt);
  P.counter = reinterpret_cast<int*>(w8);
  zero_ints_kernel<<<1, 64, 0, s>>>(P.counter, 1);
  if (a.dtype == DSA_BF16) fused_dispatch<DSA_BF16>(P, pl.grid, a.H_I / 16, s);
  else fused_dispatch<DSA_FP8_E4M3>(P, pl.grid, a.H_I / 16, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (pl.S > 1) {
    const int rows = a.B * a.Lq;
    merge_segments_kernel<<<(rows + 3) / 4, 256, 0, s>>>(P.seg_out, P.seg_cnt, rows, pl.S, k, idx);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace dsa
