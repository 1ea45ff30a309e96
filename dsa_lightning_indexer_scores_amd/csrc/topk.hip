// Deterministic top-k over materialised score rows (gfx950).
//
// GLM-5.2 技术报告速览, section "IndexShare": keep the k highest indexer scores of each
// query; GLM-5 technical report, section 3.2, paragraph "DSA RL 要点": the top-k operator must be
// deterministic.
//
// One workgroup per row.  Scores are mapped to order-preserving uint32 keys.  From a
// 2048-bin histogram of the top 11 key bits (built by the score kernel, or by one pass
// here) the workgroup finds the digit d1 of the k-th largest key.  A single streaming
// read of the row then compacts, in position order, every entry whose digit is >= d1
// into an LDS list (block-wide prefix sums keep the order); the exact k-th key theta is
// radix-selected on the list's lower 21 bits in LDS, and a final ordered pass emits the
// keys > theta plus the first needed keys == theta.  The output is therefore in
// ascending position order and identical from run to run.  When the digit's bin is too
// large for LDS, the row is processed with the same selection rule directly in global
// memory (radix passes over the row, then an ordered emitting pass).
#include "dsa_common.hpp"
#include "dsa_launch.hpp"
#include "../../include/dsa.h"

namespace dsa {

constexpr int kTopBins = 2048;          // histogram of key bits [31:21]
constexpr int kTopBS = 1024;            // threads per row
constexpr int kListCap = 8192;          // LDS candidate list (keys + positions: 64 KB)

// Block-wide exclusive prefix of v (position order = thread order); returns the prefix
// and writes the block total.  sh: scratch of kTopBS/64 words.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kTopBS / 64; ++i) {
    const uint32_t c = sh[i];
    if (i < w) before += c;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
}

// Digit d (0..nb-1) of the krem-th largest entry of an LDS histogram: count(> d) < krem
// <= count(>= d).  Block-wide; returns d and count(> d).
__device__ void block_find_digit(const uint32_t* hist, int nb, uint32_t krem, uint32_t* sh, uint32_t& d,
                                 uint32_t& above) {
  // each thread owns bins [tid*per, tid*per + per) ; suffix sums over threads
  const int per = nb / kTopBS;  // 2 for 2048 bins, 1 for 1024
  const int tid = threadIdx.x;
  uint32_t tot = 0;
  for (int j = 0; j < per; ++j) tot += hist[tid * per + j];
  // suffix = total - inclusive prefix + tot
  uint32_t all;
  const uint32_t excl = block_excl_scan(tot, sh, all);
  const uint32_t above_thread = all - excl - tot;   // entries in bins of higher threads
  if (above_thread < krem && above_thread + tot >= krem) {
    uint32_t c = above_thread;
    int dd = tid * per;
    for (int j = per - 1; j >= 0; --j) {
      const uint32_t h = hist[tid * per + j];
      if (c + h >= krem) { dd = tid * per + j; break; }
      c += h;
    }
    sh[kTopBS / 64] = (uint32_t)dd;
    sh[kTopBS / 64 + 1] = c;
  }
  __syncthreads();
  d = sh[kTopBS / 64];
  above = sh[kTopBS / 64 + 1];
  __syncthreads();
}

// Number of valid entries of a row (explicit counts, or the causal rule of the indexer).
__device__ __forceinline__ int row_valid(int row, int n, const int32_t* n_valid, int causal_Lq, int causal_Lk) {
  int nv = n;
  if (n_valid) nv = n_valid[row];
  else if (causal_Lq > 0) nv = causal_Lk - causal_Lq + (row % causal_Lq) + 1;
  return max(0, min(nv, n));
}

// Rows with at most k valid entries select all of them, padded with -1.
__device__ void emit_short_row(const float* x, int nv, int k, int32_t* out, float* vout) {
  for (int j = threadIdx.x; j < k; j += kTopBS) {
    out[j] = j < nv ? j : -1;
    if (vout) vout[j] = j < nv ? x[j] : -INFINITY;
  }
}

// Top-11-bit histogram of the row (from row_hist or one pass) and the digit d1 of the
// k-th largest key with a1 = count(digit > d1), h1 = count(digit == d1).
__device__ void row_top_digit(const float* x, int nv, int row, const uint32_t* row_hist, int k, uint32_t* hist,
                              uint32_t* sh, uint32_t& d1, uint32_t& a1, uint32_t& h1) {
  const int tid = threadIdx.x;
  if (row_hist) {
    for (int j = tid; j < kTopBins; j += kTopBS) hist[j] = row_hist[(size_t)row * kTopBins + j];
  } else {
    for (int j = tid; j < kTopBins; j += kTopBS) hist[j] = 0;
    __syncthreads();
    for (int e = tid; e < nv; e += kTopBS) atomicAdd(&hist[order_key(x[e]) >> 21], 1u);
  }
  __syncthreads();
  block_find_digit(hist, kTopBins, (uint32_t)k, sh, d1, a1);
  h1 = hist[d1];
  __syncthreads();
}

// One streaming pass over x[lo, hi) appending, in position order, every entry with
// score >= fmin (order-key digit >= d1) to ok/op (LDS or global, at most cap entries by
// construction).  A chunk is 16 sub-chunks of kTopBS consecutive entries (coalesced
// loads); entry (u, tid) goes to slot base + prefix over (sub-chunk, wave) of the kept
// counts + its rank among the wave's kept entries.  The next chunk's loads are issued
// before the current chunk is compacted.  Returns the number appended.
template <typename KeyPtr>
__device__ uint32_t collect_range(const float* x, int lo, int hi, float fmin, KeyPtr ok, KeyPtr op, uint32_t cap,
                                  uint32_t* wtot, uint32_t* sh) {
  constexpr int kSub = 16;
  constexpr int kChunk = kTopBS * kSub;
  constexpr int kNW = kTopBS / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t base = 0;
  float cur[kSub], nxt[kSub];
  auto load_chunk = [&](int c0, float (&v)[kSub]) {
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      const int e = c0 + u * kTopBS + tid;
      v[u] = e < hi ? x[e] : -INFINITY;
    }
  };
  load_chunk(lo, cur);
  for (int c0 = lo; c0 < hi; c0 += kChunk) {
    if (c0 + kChunk < hi) load_chunk(c0 + kChunk, nxt);
    uint64_t m[kSub];
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      const int e = c0 + u * kTopBS + tid;
      m[u] = ballot(e < hi && cur[u] >= fmin);
      if (lane == 0) wtot[u * kNW + w] = (uint32_t)popc64(m[u]);
    }
    __syncthreads();
    if (w == 0) {  // exclusive prefix of the kSub*kNW counts (4 per lane), in position order
      uint32_t c[4], t = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { c[i] = wtot[4 * lane + i]; t += c[i]; }
      uint32_t incl = t;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
      }
      uint32_t run = incl - t;
#pragma unroll
      for (int i = 0; i < 4; ++i) { wtot[4 * lane + i] = run; run += c[i]; }
      if (lane == 63) sh[0] = incl;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      if (m[u] == 0) continue;   // wave-uniform: nothing kept in this sub-chunk
      if ((m[u] >> lane) & 1ull) {
        const uint32_t o = base + wtot[u * kNW + w] + rank_below(m[u]);
        const int e = c0 + u * kTopBS + tid;
        if (o < cap) {   // holds by construction
          ok[o] = order_key(cur[u]);
          op[o] = (uint32_t)e;
        }
      }
    }
    base += sh[0];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSub; ++u) cur[u] = nxt[u];
  }
  return base;
}

// Exact selection on an LDS list of the nl entries with digit >= d1 (position order):
// the remaining k - a1 among digit d1 are found on bits [20:0], then the keys > theta
// and the first needed keys == theta are emitted in list (= position) order.
__device__ void select_emit_list(const uint32_t* lkeys, const uint32_t* lpos, uint32_t nl, uint32_t d1, uint32_t a1,
                                 int k, const float* x, uint32_t* hist, uint32_t* sh, int32_t* out, float* vout) {
  const int tid = threadIdx.x;
  uint32_t krem = (uint32_t)k - a1, d2, a2, d3, a3;
  for (int j = tid; j < kTopBins; j += kTopBS) hist[j] = 0;
  __syncthreads();
  for (uint32_t e = tid; e < nl; e += kTopBS)
    if ((lkeys[e] >> 21) == d1) atomicAdd(&hist[(lkeys[e] >> 10) & 0x7FFu], 1u);
  __syncthreads();
  block_find_digit(hist, kTopBins, krem, sh, d2, a2);
  krem -= a2;
  const uint32_t pre = (d1 << 21) | (d2 << 10);
  for (int j = tid; j < kTopBins; j += kTopBS) hist[j] = 0;
  __syncthreads();
  for (uint32_t e = tid; e < nl; e += kTopBS)
    if ((lkeys[e] >> 10) == (pre >> 10)) atomicAdd(&hist[lkeys[e] & 0x3FFu], 1u);
  __syncthreads();
  block_find_digit(hist, kTopBins, krem, sh, d3, a3);
  const uint32_t theta = pre | d3;
  const uint32_t need_eq = krem - a3;
  uint32_t out_n = 0, eq_seen = 0;
  for (uint32_t c0 = 0; c0 < nl; c0 += kTopBS) {
    const uint32_t e = c0 + tid;
    const bool v = e < nl;
    const uint32_t key = v ? lkeys[e] : 0u;
    const bool gt = v && key > theta, eq = v && key == theta;
    uint32_t eq_tot;
    const uint32_t eq_before = eq_seen + block_excl_scan(eq ? 1u : 0u, sh, eq_tot);
    const bool take = gt || (eq && eq_before < need_eq);
    uint32_t t_tot;
    const uint32_t pos = out_n + block_excl_scan(take ? 1u : 0u, sh, t_tot);
    if (take) {
      out[pos] = (int32_t)lpos[e];
      if (vout) vout[pos] = x[lpos[e]];
    }
    out_n += t_tot;
    eq_seen += eq_tot;
  }
}

// The selection rule applied directly on the row (when the digit's bin is too large for
// the LDS list): two more radix passes over the row, then an ordered emitting pass.
__device__ void select_emit_row(const float* x, int nv, uint32_t d1, uint32_t a1, int k, uint32_t* hist,
                                uint32_t* sh, int32_t* out, float* vout) {
  const int tid = threadIdx.x;
  uint32_t prefix = d1 << 21, pmask = 0x7FFu << 21, krem = (uint32_t)k - a1, d, above;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    const uint32_t dmask = pass == 0 ? 0x7FFu : 0x3FFu;
    for (int j = tid; j < kTopBins; j += kTopBS) hist[j] = 0;
    __syncthreads();
    for (int e = tid; e < nv; e += kTopBS) {
      const uint32_t key = order_key(x[e]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    block_find_digit(hist, kTopBins, krem, sh, d, above);
    prefix |= d << shift;
    pmask |= dmask << shift;
    krem -= above;
  }
  const uint32_t theta = prefix, need_eq = krem;
  uint32_t out_n = 0, eq_seen = 0;
  for (int c0 = 0; c0 < nv && out_n < (uint32_t)k; c0 += kTopBS) {
    const int e = c0 + tid;
    const bool v = e < nv;
    const float xv = v ? x[e] : 0.f;
    const uint32_t key = v ? order_key(xv) : 0u;
    const bool gt = v && key > theta, eq = v && key == theta;
    uint32_t eq_tot;
    const uint32_t eq_before = eq_seen + block_excl_scan(eq ? 1u : 0u, sh, eq_tot);
    const bool take = gt || (eq && eq_before < need_eq);
    uint32_t t_tot;
    const uint32_t pos = out_n + block_excl_scan(take ? 1u : 0u, sh, t_tot);
    if (take) {
      out[pos] = e;
      if (vout) vout[pos] = xv;
    }
    out_n += t_tot;
    eq_seen += eq_tot;
  }
}

// Whole row in one workgroup.
__global__ __launch_bounds__(kTopBS) void topk_rows_kernel(const float* __restrict__ scores, int64_t row_stride,
                                                          int n, const int32_t* __restrict__ n_valid,
                                                          int causal_Lq, int causal_Lk,
                                                          const uint32_t* __restrict__ row_hist, int k,
                                                          int32_t* __restrict__ idx, float* __restrict__ vals) {
  __shared__ uint32_t hist[kTopBins];
  __shared__ uint32_t lkeys[kListCap];
  __shared__ uint32_t lpos[kListCap];
  __shared__ uint32_t sh[kTopBS / 64 + 2];
  __shared__ uint32_t wtot[16 * (kTopBS / 64)];
  const int row = blockIdx.x;
  const float* x = scores + (size_t)row * row_stride;
  const int nv = row_valid(row, n, n_valid, causal_Lq, causal_Lk);
  int32_t* out = idx + (size_t)row * k;
  float* vout = vals ? vals + (size_t)row * k : nullptr;
  if (nv <= k) {
    emit_short_row(x, nv, k, out, vout);
    return;
  }
  uint32_t d1, a1, h1;
  row_top_digit(x, nv, row, row_hist, k, hist, sh, d1, a1, h1);
  if (a1 + h1 <= (uint32_t)kListCap) {
    const uint32_t nl = collect_range(x, 0, nv, key_to_float(d1 << 21), lkeys, lpos, (uint32_t)kListCap, wtot, sh);
    __syncthreads();
    select_emit_list(lkeys, lpos, min(nl, (uint32_t)kListCap), d1, a1, k, x, hist, sh, out, vout);
  } else {
    select_emit_row(x, nv, d1, a1, k, hist, sh, out, vout);
  }
}

// Few long rows: the row is split into P ranges.  topk_collect_kernel (grid P x rows)
// appends each range's candidates (digit >= d1, position order) to its own slot of the
// scratch lists; topk_finish_kernel (one workgroup per row) concatenates the P lists in
// range order into LDS and selects exactly there.  Same selection rule and output as
// topk_rows_kernel.
struct TopkSplit {
  int P, chunk;        // ranges per row, entries per range
  uint32_t cap;        // list slots per range
  uint32_t* keys;      // [rows][P][cap]
  uint32_t* pos;       // [rows][P][cap]
  uint32_t* cnt;       // [rows][P]
};

__global__ __launch_bounds__(kTopBS) void topk_collect_kernel(const float* __restrict__ scores, int64_t row_stride,
                                                             int n, const int32_t* __restrict__ n_valid,
                                                             int causal_Lq, int causal_Lk,
                                                             const uint32_t* __restrict__ row_hist, int k,
                                                             TopkSplit T) {
  __shared__ uint32_t hist[kTopBins];
  __shared__ uint32_t sh[kTopBS / 64 + 2];
  __shared__ uint32_t wtot[16 * (kTopBS / 64)];
  const int row = blockIdx.y, c = blockIdx.x;
  const float* x = scores + (size_t)row * row_stride;
  const int nv = row_valid(row, n, n_valid, causal_Lq, causal_Lk);
  uint32_t got = 0;
  if (nv > k) {
    uint32_t d1, a1, h1;
    row_top_digit(x, nv, row, row_hist, k, hist, sh, d1, a1, h1);
    if (a1 + h1 <= (uint32_t)kListCap) {
      const int lo = min(nv, c * T.chunk), hi = min(nv, lo + T.chunk);
      const size_t slot = ((size_t)row * T.P + c) * T.cap;
      got = collect_range(x, lo, hi, key_to_float(d1 << 21), T.keys + slot, T.pos + slot, T.cap, wtot, sh);
    }
  }
  if (threadIdx.x == 0) T.cnt[(size_t)row * T.P + c] = got;
}

__global__ __launch_bounds__(kTopBS) void topk_finish_kernel(const float* __restrict__ scores, int64_t row_stride,
                                                            int n, const int32_t* __restrict__ n_valid,
                                                            int causal_Lq, int causal_Lk,
                                                            const uint32_t* __restrict__ row_hist, int k,
                                                            TopkSplit T, int32_t* __restrict__ idx,
                                                            float* __restrict__ vals) {
  __shared__ uint32_t hist[kTopBins];
  __shared__ uint32_t lkeys[kListCap];
  __shared__ uint32_t lpos[kListCap];
  __shared__ uint32_t sh[kTopBS / 64 + 2];
  const int row = blockIdx.x, tid = threadIdx.x;
  const float* x = scores + (size_t)row * row_stride;
  const int nv = row_valid(row, n, n_valid, causal_Lq, causal_Lk);
  int32_t* out = idx + (size_t)row * k;
  float* vout = vals ? vals + (size_t)row * k : nullptr;
  if (nv <= k) {
    emit_short_row(x, nv, k, out, vout);
    return;
  }
  uint32_t d1, a1, h1;
  row_top_digit(x, nv, row, row_hist, k, hist, sh, d1, a1, h1);
  if (a1 + h1 > (uint32_t)kListCap) {
    select_emit_row(x, nv, d1, a1, k, hist, sh, out, vout);
    return;
  }
  uint32_t nl = 0;
  for (int c = 0; c < T.P; ++c) {
    const uint32_t m = T.cnt[(size_t)row * T.P + c];
    const size_t slot = ((size_t)row * T.P + c) * T.cap;
    for (uint32_t j = tid; j < m; j += kTopBS) {
      if (nl + j < (uint32_t)kListCap) {   // holds by construction (sum == a1 + h1)
        lkeys[nl + j] = T.keys[slot + j];
        lpos[nl + j] = T.pos[slot + j];
      }
    }
    nl += m;
  }
  __syncthreads();
  select_emit_list(lkeys, lpos, min(nl, (uint32_t)kListCap), d1, a1, k, x, hist, sh, out, vout);
}

// Rows scored as chunk candidate lists (indexer_chunksel_kernel): the lists of a row,
// concatenated in chunk order, are in position order and hold every entry of digit >= d1
// (the row's k-th digit).  lists_filter_kernel drops their entries below d1;
// topk_lists_finish_kernel then selects exactly in LDS, or, when the entries do not fit,
// with the same rule over the lists in global memory (select_emit_lists_global).
__device__ void select_emit_lists_global(const ChunkLists& L, int row, uint32_t d1, uint32_t a1, int k,
                                         uint32_t* hist, uint32_t* sh, int32_t* out) {
  const int tid = threadIdx.x;
  uint32_t prefix = d1 << 21, pmask = 0x7FFu << 21, krem = (uint32_t)k - a1, d, above;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    const uint32_t dmask = pass == 0 ? 0x7FFu : 0x3FFu;
    for (int j = tid; j < kTopBins; j += kTopBS) hist[j] = 0;
    __syncthreads();
    for (int c = 0; c < L.n_chunks; ++c) {
      const uint32_t m = L.cnt[(size_t)row * L.n_chunks + c];
      const uint32_t* kk = L.keys + (size_t)row * L.row_stride + (size_t)c * L.chunk;
      for (uint32_t j = tid; j < m; j += kTopBS) {
        const uint32_t key = kk[j];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
      }
    }
    __syncthreads();
    block_find_digit(hist, kTopBins, krem, sh, d, above);
    prefix |= d << shift;
    pmask |= dmask << shift;
    krem -= above;
  }
  const uint32_t theta = prefix, need_eq = krem;
  uint32_t out_n = 0, eq_seen = 0;
  for (int c = 0; c < L.n_chunks; ++c) {
    const uint32_t m = L.cnt[(size_t)row * L.n_chunks + c];
    const size_t base = (size_t)row * L.row_stride + (size_t)c * L.chunk;
    for (uint32_t j0 = 0; j0 < m; j0 += kTopBS) {
      const uint32_t j = j0 + tid;
      const bool v = j < m;
      const uint32_t key = v ? L.keys[base + j] : 0u;
      const bool gt = v && key > theta, eq = v && key == theta;
      uint32_t eq_tot;
      const uint32_t eq_before = eq_seen + block_excl_scan(eq ? 1u : 0u, sh, eq_tot);
      const bool take = gt || (eq && eq_before < need_eq);
      uint32_t t_tot;
      const uint32_t o = out_n + block_excl_scan(take ? 1u : 0u, sh, t_tot);
      if (take) out[o] = (int32_t)L.pos[base + j];
      out_n += t_tot;
      eq_seen += eq_tot;
    }
  }
}

// One workgroup per row, after the filter: the lists hold exactly the row's entries of
// digit >= d1 (a1 + h1 of them), in position order once concatenated by chunk.  They are
// copied into LDS (flattened, chunk found from the offset table) and selected there;
// when they do not fit, the selection runs over the lists in global memory.
__global__ __launch_bounds__(kTopBS) void topk_lists_finish_kernel(ChunkLists L, int causal_Lq, int causal_Lk, int k,
                                                                  int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[kTopBins];
  __shared__ uint32_t lkeys[kListCap];
  __shared__ uint32_t lpos[kListCap];
  __shared__ uint32_t offs[kTopBS + 1];
  __shared__ uint32_t sh[kTopBS / 64 + 2];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int nv = max(0, chunk_lists_seq_len(L, row / causal_Lq, causal_Lk) - causal_Lq + (row % causal_Lq) + 1);
  int32_t* out = idx + (size_t)row * k;
  if (nv <= k) {
    emit_short_row(nullptr, nv, k, out, nullptr);
    return;
  }
  uint32_t d1, a1, h1;
  row_top_digit(nullptr, nv, row, L.row_hist, k, hist, sh, d1, a1, h1);
  if (a1 + h1 > (uint32_t)kListCap) {
    select_emit_lists_global(L, row, d1, a1, k, hist, sh, out);
    return;
  }
  // chunks in groups of kTopBS: offset table, then a flattened copy of the group's entries
  uint32_t nl = 0;
  for (int c0 = 0; c0 < L.n_chunks; c0 += kTopBS) {
    const int nc = min(kTopBS, L.n_chunks - c0);
    const uint32_t m = tid < nc ? L.cnt[(size_t)row * L.n_chunks + c0 + tid] : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan(m, sh, tot);
    if (tid < nc) offs[tid] = ex;
    if (tid == 0) offs[nc] = tot;
    __syncthreads();
    for (uint32_t e = tid; e < tot; e += kTopBS) {
      int lo = 0, hi = nc - 1;   // last chunk with offs[c] <= e
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offs[mid] <= e) lo = mid;
        else hi = mid - 1;
      }
      const uint32_t o = nl + e;
      if (o < (uint32_t)kListCap) {   // holds: the lists hold a1 + h1 entries
        const size_t src = (size_t)row * L.row_stride + (size_t)(c0 + lo) * L.chunk + (e - offs[lo]);
        lkeys[o] = L.keys[src];
        lpos[o] = L.pos[src];
      }
    }
    nl += tot;
    __syncthreads();
  }
  select_emit_list(lkeys, lpos, min(nl, (uint32_t)kListCap), d1, a1, k, nullptr, hist, sh, out, nullptr);
}

hipError_t launch_topk_lists_finish(const ChunkLists& L, int rows, int causal_Lq, int causal_Lk, int k,
                                    int32_t* idx, hipStream_t s) {
  topk_lists_finish_kernel<<<rows, kTopBS, 0, s>>>(L, causal_Lq, causal_Lk, k, idx);
  return hipGetLastError();
}

// Top-11-bit key histogram of each row for the split path when the score kernel did not
// provide one: each workgroup counts its range in LDS and adds the non-zero bins to the
// row's global histogram (zeroed beforehand).
__global__ __launch_bounds__(kTopBS) void topk_hist_kernel(const float* __restrict__ scores, int64_t row_stride,
                                                          int n, const int32_t* __restrict__ n_valid, int chunk,
                                                          uint32_t* __restrict__ row_hist) {
  __shared__ uint32_t hist[kTopBins];
  const int row = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const float* x = scores + (size_t)row * row_stride;
  const int nv = row_valid(row, n, n_valid, 0, 0);
  for (int j = tid; j < kTopBins; j += kTopBS) hist[j] = 0;
  __syncthreads();
  const int lo = min(nv, c * chunk), hi = min(nv, lo + chunk);
  for (int e = lo + tid; e < hi; e += kTopBS) atomicAdd(&hist[order_key(x[e]) >> 21], 1u);
  __syncthreads();
  for (int j = tid; j < kTopBins; j += kTopBS)
    if (hist[j]) atomicAdd(&row_hist[(size_t)row * kTopBins + j], hist[j]);
}

// Ranges per row for the split path (1 = single-workgroup path): enough workgroups for
// the GPU, at least 4096 entries per range.
static TopkSplit plan_topk_split(int rows, int n) {
  TopkSplit T{};
  int P = (512 + rows - 1) / rows;
  const int max_p = (n + 4095) / 4096;
  if (P > max_p) P = max_p;
  if (P < 1) P = 1;
  T.P = P;
  T.chunk = ((n + P - 1) / P + 1023) / 1024 * 1024;
  T.cap = (uint32_t)min(T.chunk, kListCap);
  return T;
}

static size_t split_lists_bytes(const TopkSplit& T, int rows) {
  return ((size_t)rows * T.P * T.cap * 2 * sizeof(uint32_t) + (size_t)rows * T.P * sizeof(uint32_t) + 255) / 256 * 256;
}

size_t topk_split_ws(int rows, int n, bool with_hist) {
  const TopkSplit T = plan_topk_split(rows, n);
  if (T.P == 1) return 0;
  return split_lists_bytes(T, rows) + (with_hist ? (size_t)rows * kTopBins * sizeof(uint32_t) : 0);
}

hipError_t launch_topk_rows(const float* scores, int64_t row_stride, int rows, int n,
                            const int32_t* n_valid, int causal_Lq, int causal_Lk, const uint32_t* row_hist,
                            int k, int32_t* idx, float* vals, void* scratch, size_t scratch_bytes, hipStream_t s) {
  TopkSplit T = plan_topk_split(rows, n);
  const size_t need = topk_split_ws(rows, n, row_hist == nullptr);
  if (T.P > 1 && scratch && scratch_bytes >= need) {
    T.keys = static_cast<uint32_t*>(scratch);
    T.pos = T.keys + (size_t)rows * T.P * T.cap;
    T.cnt = T.pos + (size_t)rows * T.P * T.cap;
    if (!row_hist) {
      uint32_t* h = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(scratch) + split_lists_bytes(T, rows));
      hipError_t e = launch_zero(h, (size_t)rows * kTopBins * sizeof(uint32_t), s);
      if (e != hipSuccess) return e;
      topk_hist_kernel<<<dim3(T.P, rows), kTopBS, 0, s>>>(scores, row_stride, n, n_valid, T.chunk, h);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      row_hist = h;
    }
    topk_collect_kernel<<<dim3(T.P, rows), kTopBS, 0, s>>>(scores, row_stride, n, n_valid, causal_Lq, causal_Lk,
                                                           row_hist, k, T);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    topk_finish_kernel<<<rows, kTopBS, 0, s>>>(scores, row_stride, n, n_valid, causal_Lq, causal_Lk, row_hist, k,
                                               T, idx, vals);
    return hipGetLastError();
  }
  topk_rows_kernel<<<rows, kTopBS, 0, s>>>(scores, row_stride, n, n_valid, causal_Lq, causal_Lk, row_hist, k,
                                           idx, vals);
  return hipGetLastError();
}

}  // namespace dsa
