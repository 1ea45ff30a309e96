// Host-side launchers of the DSA kernels (internal to libdsa.so).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace dsa {

struct IndexerArgs {
  const void* q;         // [B, Lq, H_I, d_I]
  const float* q_scale;  // [B, Lq] or null
  const void* k;         // [B, Lk, d_I]
  const float* k_scale;  // [B, Lk] or null
  const float* w;        // [B, Lq, H_I]
  int H_I, d_I, dtype;
  int B, Lq, Lk;
};

// Capacity (entries) of the per-row streaming candidate buffer of the fused kernel.
inline int topk_buffer_capacity(int k) {
  int cap = 4 * k;
  if (cap < k + 512) cap = k + 512;
  return (cap + 63) / 64 * 64;
}

// --- indexer ---------------------------------------------------------------
// scores: row r = (b, i) at scores + r * stride (stride >= Lk).
// row_hist (optional, [B*Lq][2048] uint32, zeroed by the caller): per-row histogram of
// the top 11 bits of the order keys of the causal scores.
hipError_t launch_indexer_scores(const IndexerArgs& a, float* scores, int64_t stride, uint32_t* row_hist,
                                 hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
constexpr int kRowHistBins = 2048;
// Fused streaming indexer + top-k for query counts large enough to fill the GPU.
size_t indexer_topk_fused_ws(int B, int Lq, int Lk, int k, int dtype);
hipError_t launch_indexer_topk_fused(const IndexerArgs& a, int k, int32_t* idx, void* ws,
                                     size_t ws_bytes, hipStream_t s);

// --- few query rows (decode): chunk candidate lists, then the row top-k -------
// Every (row, chunk) workgroup keeps its chunk's scores in LDS and writes, in position
// order, the entries whose top-11-bit digit is at least the chunk's own k-th digit.  The
// row's k-th key is never below any chunk's, so the lists hold every entry of the row's
// top-k; the finishing kernel filters them by the row's digit and selects exactly.
struct ChunkLists {
  int chunk;            // keys per chunk (multiple of 64)
  int n_chunks;         // chunks per row
  int64_t row_stride;   // list slots per row (>= n_chunks * chunk); chunk c at c * chunk
  uint32_t* keys;       // [rows][row_stride] order keys
  uint32_t* pos;        // [rows][row_stride] positions
  uint32_t* cnt;        // [rows][n_chunks] entries per list
  uint32_t* row_hist;   // [rows][2048] top-11-bit histogram of the causal scores
  const int32_t* seq_lens;  // [B] keys held by each sequence's cache (clamped to [0, Lk]), or
                            // null: every sequence holds Lk
  // paged caches (block_table null: k^I / k_scale are [B, Lk] arrays): position s of
  // sequence b is row block_table[b * max_pages + s / page] * page + s % page of the pools
  // (page ids clamped to [0, pool_pages)); page is a power of two, a multiple of 64
  const int32_t* block_table;
  int max_pages, page_log2, pool_pages;
};
// Keys of sequence b (device side): seq_lens[b] clamped to [0, Lk], or Lk.
__device__ __forceinline__ int chunk_lists_seq_len(const ChunkLists& L, int b, int Lk) {
  return L.seq_lens ? min(max(L.seq_lens[b], 0), Lk) : Lk;
}
size_t chunk_lists_ws(int rows, int Lk);
struct PagedCache {
  const int32_t* block_table;   // null: contiguous [B, Lk] caches
  int max_pages, page_log2, pool_pages;
};
hipError_t launch_indexer_topk_lists(const IndexerArgs& a, int k, const int32_t* seq_lens, const PagedCache& pc,
                                     int32_t* idx, void* ws, size_t ws_bytes, hipStream_t s);
// idx positions of a paged batch -> physical pool rows (-1 for -1 and out-of-range entries)
hipError_t launch_paged_rows(const int32_t* idx, int B, int Lq, int k, const PagedCache& pc, int32_t* rows_out,
                             hipStream_t s);
hipError_t launch_topk_lists_finish(const ChunkLists& L, int rows, int causal_Lq, int causal_Lk, int k,
                                    int32_t* idx, hipStream_t s);

// --- top-k over materialised rows -------------------------------------------
// With scratch of at least topk_split_ws(rows, n, row_hist == nullptr) bytes, few long
// rows are split over several workgroups; otherwise one workgroup handles a row.
size_t topk_split_ws(int rows, int n, bool with_hist);
hipError_t launch_topk_rows(const float* scores, int64_t row_stride, int rows, int n,
                            const int32_t* n_valid, int causal_Lq, int causal_Lk, const uint32_t* row_hist,
                            int k, int32_t* idx, float* vals, void* scratch, size_t scratch_bytes, hipStream_t s);

// --- per-token E4M3 quantization ---------------------------------------------
// rows of row_elems values (fp32 or bf16, row r at x + r * x_stride elements) -> codes at
// codes + r * c_stride bytes and scales[r * s_stride].
hipError_t launch_quantize_e4m3(const void* x, int x_dtype, int rows, int row_elems, int64_t x_stride,
                                uint8_t* codes, int64_t c_stride, float* scales, int64_t s_stride, hipStream_t s);

// --- bf16 linear map (indexer projections): y[M, N] fp32 = x[M, K] . w[N, K]^T ----
hipError_t launch_linear_bf16(const void* x, int64_t ldx, const void* w, int64_t ldw, int M, int N, int K, float* y,
                              int64_t ldy, hipStream_t s);

// --- group-centroid objective of the indexer (training) ------------------------
struct AttnProbsArgs {
  const void* q;            // [B, Lq, H, 576] bf16
  const void* kv;           // latent rows, [B, Lk] rows of k_row_stride bf16 (first 576 used)
  int64_t k_row_stride;
  const float* lse;         // [B, Lq, H] natural-log sum of exp(sm_scale q . K) over the row
  const int32_t* idx;       // row r at idx + r * idx_q_stride, k entries
  int64_t idx_q_stride;
  float* P;                 // [B, Lq, k], accumulated
  float sm_scale, alpha;
  int B, Lq, Lk, H, k;
};
hipError_t launch_attn_probs(const AttnProbsArgs& a, hipStream_t s);
constexpr int kMaxKlK = 2048;   // index-row length limit of the backward (its scores stay in LDS)
struct IndexerKlArgs {
  const void* q;            // [B, Lq, H_I, 128] bf16
  const void* kI;           // [B, Lk, 128] bf16
  const float* w;           // [B, Lq, H_I]
  const int32_t* idx;       // [B, Lq, k]
  const float* pbar;        // [B, Lq, k]
  float* loss;              // [B, Lq]
  float* dq;                // [B, Lq, H_I, 128]
  float* dw;                // [B, Lq, H_I]
  float* dk;                // [B, Lk, 128], added to
  unsigned long long* dk_fix;  // [B, Lk, 128] 64-bit fixed-point sums (workspace)
  int B, Lq, Lk, H_I, k;
};
// dk contributions are rounded to multiples of 2^-kDkFixBits and summed as 64-bit integers,
// so the result does not depend on the order in which rows add them
constexpr int kDkFixBits = 30;
inline size_t indexer_kl_ws(int B, int Lk) { return ((size_t)B * Lk * 128 * 8 + 255) / 256 * 256; }
hipError_t launch_indexer_kl(const IndexerKlArgs& a, hipStream_t s);

// --- sparse attention --------------------------------------------------------
struct AttnArgs {
  const void* q;
  const void* k;
  int64_t k_row_stride;
  const void* v;
  int64_t v_row_stride;
  void* out;
  float* lse;
  int H, Hkv, Dqk, Dv;
  float sm_scale;
  int dtype;
  int out_dtype;
  int B, Lq, Lk;
  const int32_t* idx;
  int64_t idx_q_stride;
  int topk;          // entries per idx row
  int kv8;           // latent rows are E4M3 codes (k_row_stride in bytes) ...
  const float* kv_scale;   // ... with one fp32 scale per row, [B, Lk]
};
size_t sparse_attn_ws(int B, int Lq, int k, int H, int64_t idx_q_stride, int dtype);
hipError_t launch_sparse_attn(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s);

}  // namespace dsa
