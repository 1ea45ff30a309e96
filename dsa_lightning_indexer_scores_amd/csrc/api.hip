// C ABI of libdsa.so: argument validation, workspace planning and dispatch.
// Every check runs on the host before anything is enqueued; see include/dsa.h.
#include "../../include/dsa.h"
#include "dsa_launch.hpp"

#include <stdint.h>

#include <mutex>

// Device buffer of dsa_sparse_attn_noalloc (split-key partial results), one copy on each
// GPU the library runs on.  Host code never uses this name as an address: the device
// address of each GPU's copy is looked up once (noalloc_scratch below) and passed on.
static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxFusedK = 4096;
constexpr int kMaxTopkK = 65536;
constexpr int kMinFusedLq = 16;   // fewer queries per sequence: score rows + row top-k

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
size_t round_up(size_t x) { return (x + 255) / 256 * 256; }

bool use_materialised(int dtype, int Lq) { return dtype == DSA_F32 || Lq < kMinFusedLq; }

int check_indexer(const dsa_indexer_in* in, int B, int Lq, int Lk) {
  if (!in || !in->q || !in->k || !in->w) return DSA_ERR_ARG;
  if (B <= 0 || Lq <= 0 || Lk <= 0 || Lq > Lk) return DSA_ERR_ARG;
  switch (in->dtype) {
    case DSA_F32:
      if (in->H_I <= 0 || in->H_I > 64 || in->d_I <= 0 || (int64_t)in->H_I * in->d_I > 8192) return DSA_ERR_SHAPE;
      if (!aligned(in->q, 4) || !aligned(in->k, 4) || !aligned(in->w, 4)) return DSA_ERR_ALIGN;
      break;
    case DSA_BF16:
    case DSA_FP8_E4M3:
      if (in->H_I < 16 || in->H_I > 64 || (in->H_I % 16) != 0 || in->d_I != 128) return DSA_ERR_SHAPE;
      if (!aligned(in->q, 16) || !aligned(in->k, 16) || !aligned(in->w, 16)) return DSA_ERR_ALIGN;
      if (in->dtype == DSA_FP8_E4M3 && (!in->q_scale || !in->k_scale)) return DSA_ERR_ARG;
      break;
    default:
      return DSA_ERR_DTYPE;
  }
  return DSA_OK;
}

int check_attn(const dsa_attn_in* in, int B, int Lq, int Lk, const int32_t* idx, int64_t idx_q_stride, int k) {
  if (!in || !in->q || !in->k || !in->v || !in->out || !idx) return DSA_ERR_ARG;
  if (B <= 0 || Lq <= 0 || Lk <= 0 || k <= 0) return DSA_ERR_ARG;
  if (idx_q_stride != 0 && idx_q_stride < k) return DSA_ERR_ARG;
  if (!aligned(idx, 4) || (in->lse && !aligned(in->lse, 4))) return DSA_ERR_ALIGN;
  if (in->out_dtype != DSA_F32 && in->out_dtype != in->dtype) return DSA_ERR_DTYPE;
  switch (in->dtype) {
    case DSA_BF16:
      if (in->H < 16 || in->H > 64 || (in->H % 16) != 0 || in->Hkv != 1 || in->Dqk != 576 || in->Dv != 512)
        return DSA_ERR_SHAPE;
      if (in->v != in->k || in->v_row_stride != in->k_row_stride) return DSA_ERR_SHAPE;
      if (in->k_row_stride < 576 || (in->k_row_stride % 8) != 0) return DSA_ERR_ALIGN;
      if (!aligned(in->q, 16) || !aligned(in->k, 16) || !aligned(in->out, 16)) return DSA_ERR_ALIGN;
      break;
    case DSA_F32:
      if (in->H <= 0 || in->Hkv <= 0 || (in->H % in->Hkv) != 0 || in->Dqk <= 0 || in->Dv <= 0 ||
          in->Dqk > 256 || in->Dv > 256 || k > 8192)
        return DSA_ERR_SHAPE;
      if (in->k_row_stride < (int64_t)in->Hkv * in->Dqk || in->v_row_stride < (int64_t)in->Hkv * in->Dv)
        return DSA_ERR_SHAPE;
      if (!aligned(in->q, 4) || !aligned(in->k, 4) || !aligned(in->v, 4) || !aligned(in->out, 4)) return DSA_ERR_ALIGN;
      break;
    default:
      return DSA_ERR_DTYPE;
  }
  return DSA_OK;
}

dsa::IndexerArgs make_indexer_args(const dsa_indexer_in* in, int B, int Lq, int Lk) {
  dsa::IndexerArgs a;
  a.q = in->q;
  a.q_scale = in->q_scale;
  a.k = in->k;
  a.k_scale = in->k_scale;
  a.w = in->w;
  a.H_I = in->H_I;
  a.d_I = in->d_I;
  a.dtype = in->dtype;
  a.B = B;
  a.Lq = Lq;
  a.Lk = Lk;
  return a;
}

dsa::AttnArgs make_attn_args(const dsa_attn_in* in, int B, int Lq, int Lk, const int32_t* idx,
                             int64_t idx_q_stride, int k) {
  dsa::AttnArgs a;
  a.q = in->q;
  a.k = in->k;
  a.k_row_stride = in->k_row_stride;
  a.v = in->v;
  a.v_row_stride = in->v_row_stride;
  a.out = in->out;
  a.lse = in->lse;
  a.H = in->H;
  a.Hkv = in->Hkv;
  a.Dqk = in->Dqk;
  a.Dv = in->Dv;
  a.sm_scale = in->sm_scale;
  a.dtype = in->dtype;
  a.out_dtype = in->out_dtype;
  a.B = B;
  a.Lq = Lq;
  a.Lk = Lk;
  a.idx = idx;
  a.idx_q_stride = idx_q_stride;
  a.topk = k;
  a.kv8 = 0;
  a.kv_scale = nullptr;
  return a;
}

// materialised score rows start on 256-byte boundaries (whole-line stores)
int64_t score_stride(int Lk) { return ((int64_t)Lk + 63) / 64 * 64; }
size_t materialised_scores_bytes(int B, int Lq, int Lk) { return round_up((size_t)B * Lq * score_stride(Lk) * sizeof(float)); }
size_t materialised_hist_bytes(int B, int Lq) { return round_up((size_t)B * Lq * dsa::kRowHistBins * sizeof(uint32_t)); }

size_t indexer_topk_ws(int dtype, int B, int Lq, int Lk, int k) {
  if (dtype == DSA_F32)
    return materialised_scores_bytes(B, Lq, Lk) + materialised_hist_bytes(B, Lq) +
           round_up(dsa::topk_split_ws(B * Lq, Lk, false));
  if (use_materialised(dtype, Lq)) return round_up(dsa::chunk_lists_ws(B * Lq, Lk));
  return dsa::indexer_topk_fused_ws(B, Lq, Lk, k, dtype);
}

size_t attn_ws(int dtype, int B, int Lq, int k, int H) {
  const size_t a = dsa::sparse_attn_ws(B, Lq, k, H, (int64_t)k, dtype);
  const size_t b = dsa::sparse_attn_ws(B, Lq, k, H, 0, dtype);
  return a > b ? a : b;
}

int run_indexer_topk(const dsa_indexer_in* in, int B, int Lq, int Lk, int k, int32_t* idx, void* ws,
                     size_t ws_bytes, hipStream_t s) {
  const dsa::IndexerArgs a = make_indexer_args(in, B, Lq, Lk);
  hipError_t e;
  if (in->dtype != DSA_F32 && use_materialised(in->dtype, Lq)) {
    // few queries (decode): chunk candidate lists, no score rows
    e = dsa::launch_indexer_topk_lists(a, k, nullptr, dsa::PagedCache{}, idx, ws, ws_bytes, s);
  } else if (use_materialised(in->dtype, Lq)) {
    uint8_t* w8 = static_cast<uint8_t*>(ws);
    float* scores = reinterpret_cast<float*>(w8);
    const size_t off_hist = materialised_scores_bytes(B, Lq, Lk);
    const size_t off_split = off_hist + materialised_hist_bytes(B, Lq);
    uint32_t* hist = reinterpret_cast<uint32_t*>(w8 + off_hist);
    e = dsa::launch_zero(hist, materialised_hist_bytes(B, Lq), s);
    if (e == hipSuccess) e = dsa::launch_indexer_scores(a, scores, score_stride(Lk), hist, s);
    if (e == hipSuccess)
      e = dsa::launch_topk_rows(scores, score_stride(Lk), B * Lq, Lk, nullptr, Lq, Lk, hist, k, idx, nullptr, w8 + off_split,
                                ws_bytes - off_split, s);
  } else {
    e = dsa::launch_indexer_topk_fused(a, k, idx, ws, ws_bytes, s);
  }
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

}  // namespace

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch` on each GPU

// The device address of the scratch buffer on the device of `stream` (the current device
// for the null stream), looked up with that device current on its first use.
int noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return DSA_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return DSA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return DSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return DSA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return DSA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return DSA_ERR_HIP;
    if (e != hipSuccess || !p) return DSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

size_t dsa_workspace_size(int op, int dtype, int B, int Lq, int Lk, int k, int heads) {
  if (B <= 0 || Lq <= 0 || Lk <= 0 || k <= 0) return 0;
  switch (op) {
    case DSA_OP_TOPK:  // optional: B * Lq rows of Lk scores
      if (k > kMaxTopkK) return 0;
      return dsa::topk_split_ws(B * Lq, Lk, true);
    case DSA_OP_INDEXER_TOPK:
      if (dtype < DSA_F32 || dtype > DSA_FP8_E4M3 || k > kMaxFusedK || Lq > Lk) return 0;
      return indexer_topk_ws(dtype, B, Lq, Lk, k);
    case DSA_OP_SPARSE_ATTN:
      if (heads <= 0 || (dtype != DSA_F32 && dtype != DSA_BF16)) return 0;
      return attn_ws(dtype, B, Lq, k, heads);
    case DSA_OP_LAYER_GROUP: {
      if (dtype < DSA_F32 || dtype > DSA_FP8_E4M3 || k > kMaxFusedK || Lq > Lk || heads <= 0) return 0;
      const size_t a = indexer_topk_ws(dtype, B, Lq, Lk, k);
      // attention dtype follows the layers; bf16 needs the (larger) split workspace
      const size_t b = attn_ws(DSA_BF16, B, Lq, k, heads);
      return a > b ? a : b;
    }
    case DSA_OP_INDEXER_KL:
      if (dtype != DSA_BF16 || k > dsa::kMaxKlK) return 0;
      return dsa::indexer_kl_ws(B, Lk);
    default:
      return 0;
  }
}

int dsa_indexer_scores(const dsa_indexer_in* in, int B, int Lq, int Lk, float* scores, void* stream) {
  int st = check_indexer(in, B, Lq, Lk);
  if (st != DSA_OK) return st;
  if (!scores) return DSA_ERR_ARG;
  if (!aligned(scores, 4)) return DSA_ERR_ALIGN;
  const hipError_t e = dsa::launch_indexer_scores(make_indexer_args(in, B, Lq, Lk), scores, Lk, nullptr,
                                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

int dsa_topk(const float* scores, int64_t row_stride, int rows, int n, const int32_t* n_valid, int k,
             int32_t* idx, float* vals, void* ws, size_t ws_bytes, void* stream) {
  if (!scores || !idx) return DSA_ERR_ARG;
  if (rows <= 0 || n <= 0 || k <= 0 || k > kMaxTopkK || row_stride < n) return DSA_ERR_ARG;
  if (!aligned(scores, 4) || !aligned(idx, 4) || (vals && !aligned(vals, 4)) || (n_valid && !aligned(n_valid, 4)))
    return DSA_ERR_ALIGN;
  if (ws && !aligned(ws, 256)) return DSA_ERR_ALIGN;
  const hipError_t e = dsa::launch_topk_rows(scores, row_stride, rows, n, n_valid, 0, 0, nullptr, k, idx, vals,
                                             ws, ws ? ws_bytes : 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

int dsa_indexer_topk(const dsa_indexer_in* in, int B, int Lq, int Lk, int k, int32_t* idx, void* ws,
                     size_t ws_bytes, void* stream) {
  int st = check_indexer(in, B, Lq, Lk);
  if (st != DSA_OK) return st;
  if (!idx || k <= 0 || k > kMaxFusedK) return DSA_ERR_ARG;
  if (!aligned(idx, 4)) return DSA_ERR_ALIGN;
  const size_t need = indexer_topk_ws(in->dtype, B, Lq, Lk, k);
  if (need > 0 && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  if (ws && !aligned(ws, 256)) return DSA_ERR_ALIGN;
  return run_indexer_topk(in, B, Lq, Lk, k, idx, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

int dsa_indexer_topk_varlen(const dsa_indexer_in* in, int B, int Lq, int Lk_max, const int32_t* seq_lens, int k,
                            int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  int st = check_indexer(in, B, Lq, Lk_max);
  if (st != DSA_OK) return st;
  if (!seq_lens || !idx || k <= 0 || k > kMaxFusedK) return DSA_ERR_ARG;
  if (in->dtype == DSA_F32) return DSA_ERR_DTYPE;
  if (Lq >= kMinFusedLq) return DSA_ERR_SHAPE;
  if (!aligned(idx, 4) || !aligned(seq_lens, 4)) return DSA_ERR_ALIGN;
  const size_t need = indexer_topk_ws(in->dtype, B, Lq, Lk_max, k);
  if (!ws || ws_bytes < need) return DSA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return DSA_ERR_ALIGN;
  const hipError_t e = dsa::launch_indexer_topk_lists(make_indexer_args(in, B, Lq, Lk_max), k, seq_lens,
                                                      dsa::PagedCache{}, idx, ws, ws_bytes,
                                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

namespace {
// page_size: a power of two, a multiple of 64, at most 2^20; returns log2 or -1
int page_log2_of(int page_size) {
  if (page_size < 64 || page_size > (1 << 20) || (page_size & (page_size - 1))) return -1;
  int l = 0;
  while ((1 << l) < page_size) ++l;
  return l;
}
}  // namespace

int dsa_indexer_topk_paged(const dsa_indexer_in* in, int B, int Lq, const int32_t* seq_lens,
                           const int32_t* block_table, int max_pages, int page_size, int pool_pages, int k,
                           int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  if (!in || !block_table || !seq_lens || max_pages <= 0 || pool_pages <= 0) return DSA_ERR_ARG;
  const int lp = page_log2_of(page_size);
  if (lp < 0 || (int64_t)max_pages * page_size > (int64_t)1 << 30 || (int64_t)pool_pages * page_size > (int64_t)1 << 30)
    return DSA_ERR_SHAPE;
  const int Lk_max = max_pages * page_size;
  int st = check_indexer(in, B, Lq, Lk_max);
  if (st != DSA_OK) return st;
  if (!idx || k <= 0 || k > kMaxFusedK) return DSA_ERR_ARG;
  if (in->dtype == DSA_F32) return DSA_ERR_DTYPE;
  if (Lq >= kMinFusedLq) return DSA_ERR_SHAPE;
  if (!aligned(idx, 4) || !aligned(seq_lens, 4) || !aligned(block_table, 4)) return DSA_ERR_ALIGN;
  const size_t need = indexer_topk_ws(in->dtype, B, Lq, Lk_max, k);
  if (!ws || ws_bytes < need) return DSA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return DSA_ERR_ALIGN;
  const dsa::PagedCache pc{block_table, max_pages, lp, pool_pages};
  const hipError_t e = dsa::launch_indexer_topk_lists(make_indexer_args(in, B, Lq, Lk_max), k, seq_lens, pc, idx,
                                                      ws, ws_bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

int dsa_paged_rows(const int32_t* idx, int B, int Lq, int k, const int32_t* block_table, int max_pages,
                   int page_size, int pool_pages, int32_t* rows_out, void* stream) {
  if (!idx || !block_table || !rows_out || B <= 0 || Lq <= 0 || k <= 0 || max_pages <= 0 || pool_pages <= 0)
    return DSA_ERR_ARG;
  const int lp = page_log2_of(page_size);
  if (lp < 0 || (int64_t)max_pages * page_size > (int64_t)1 << 30 || (int64_t)pool_pages * page_size > (int64_t)1 << 30)
    return DSA_ERR_SHAPE;
  if (!aligned(idx, 4) || !aligned(block_table, 4) || !aligned(rows_out, 4)) return DSA_ERR_ALIGN;
  const dsa::PagedCache pc{block_table, max_pages, lp, pool_pages};
  const hipError_t e = dsa::launch_paged_rows(idx, B, Lq, k, pc, rows_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

int dsa_sparse_attn(const dsa_attn_in* in, int B, int Lq, int Lk, const int32_t* idx, int64_t idx_q_stride, int k,
                    void* ws, size_t ws_bytes, void* stream) {
  int st = check_attn(in, B, Lq, Lk, idx, idx_q_stride, k);
  if (st != DSA_OK) return st;
  const size_t need = dsa::sparse_attn_ws(B, Lq, k, in->H, idx_q_stride, in->dtype);
  if (need > 0 && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  if (ws && !aligned(ws, 256)) return DSA_ERR_ALIGN;
  const hipError_t e = dsa::launch_sparse_attn(make_attn_args(in, B, Lq, Lk, idx, idx_q_stride, k), ws, ws_bytes,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

int dsa_sparse_attn_noalloc(const dsa_attn_in* in, int B, int Lq, int Lk, const int32_t* idx, int64_t idx_q_stride,
                            int k, void* stream) {
  int st = check_attn(in, B, Lq, Lk, idx, idx_q_stride, k);
  if (st != DSA_OK) return st;
  const size_t need = dsa::sparse_attn_ws(B, Lq, k, in->H, idx_q_stride, in->dtype);
  if (need > DSA_NOALLOC_SCRATCH_BYTES) return DSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    st = noalloc_scratch(static_cast<hipStream_t>(stream), &ws);
    if (st != DSA_OK) return st;
  }
  const hipError_t e = dsa::launch_sparse_attn(make_attn_args(in, B, Lq, Lk, idx, idx_q_stride, k), ws,
                                               need > 0 ? (size_t)DSA_NOALLOC_SCRATCH_BYTES : 0,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

int dsa_sparse_attn_kv8(const dsa_attn_in* in, const float* kv_scale, int B, int Lq, int Lk, const int32_t* idx,
                        int64_t idx_q_stride, int k, void* ws, size_t ws_bytes, void* stream) {
  if (!in || !kv_scale) return DSA_ERR_ARG;
  if (in->dtype != DSA_BF16) return DSA_ERR_DTYPE;
  // the bf16 checks cover q, out, idx and the shapes; the cache rows are checked as codes
  dsa_attn_in as_bf16 = *in;
  as_bf16.k_row_stride = as_bf16.v_row_stride = 576;
  int st = check_attn(&as_bf16, B, Lq, Lk, idx, idx_q_stride, k);
  if (st != DSA_OK) return st;
  if (in->H > 32) return DSA_ERR_SHAPE;
  if (in->v != in->k || in->v_row_stride != in->k_row_stride) return DSA_ERR_SHAPE;
  if (in->k_row_stride < 576 || (in->k_row_stride % 16) != 0) return DSA_ERR_ALIGN;
  if (!aligned(kv_scale, 4)) return DSA_ERR_ALIGN;
  const size_t need = dsa::sparse_attn_ws(B, Lq, k, in->H, idx_q_stride, in->dtype);
  if (need > 0 && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  if (ws && !aligned(ws, 256)) return DSA_ERR_ALIGN;
  dsa::AttnArgs a = make_attn_args(in, B, Lq, Lk, idx, idx_q_stride, k);
  a.kv8 = 1;
  a.kv_scale = kv_scale;
  const hipError_t e = dsa::launch_sparse_attn(a, ws, ws_bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

int dsa_layer_group(const dsa_indexer_in* full, const dsa_attn_in* layers, int n_layers, int B, int Lq, int Lk,
                    int k, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  int st = check_indexer(full, B, Lq, Lk);
  if (st != DSA_OK) return st;
  if (!idx_out || k <= 0 || k > kMaxFusedK || n_layers < 0 || (n_layers > 0 && !layers)) return DSA_ERR_ARG;
  if (!aligned(idx_out, 4)) return DSA_ERR_ALIGN;
  for (int l = 0; l < n_layers; ++l) {
    st = check_attn(&layers[l], B, Lq, Lk, idx_out, (int64_t)k, k);
    if (st != DSA_OK) return st;
    if (layers[l].dtype != layers[0].dtype || layers[l].H != layers[0].H || layers[l].Dqk != layers[0].Dqk ||
        layers[l].Dv != layers[0].Dv)
      return DSA_ERR_SHAPE;
  }
  size_t need = indexer_topk_ws(full->dtype, B, Lq, Lk, k);
  for (int l = 0; l < n_layers; ++l) {
    const size_t a = dsa::sparse_attn_ws(B, Lq, k, layers[l].H, (int64_t)k, layers[l].dtype);
    if (a > need) need = a;
  }
  if (need > 0 && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  if (ws && !aligned(ws, 256)) return DSA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_indexer_topk(full, B, Lq, Lk, k, idx_out, ws, ws_bytes, s);
  if (st != DSA_OK) return st;
  for (int l = 0; l < n_layers; ++l) {
    const hipError_t e =
        dsa::launch_sparse_attn(make_attn_args(&layers[l], B, Lq, Lk, idx_out, (int64_t)k, k), ws, ws_bytes, s);
    if (e != hipSuccess) return DSA_ERR_HIP;
  }
  return DSA_OK;
}

int dsa_quantize_e4m3(const void* x, int x_dtype, int rows, int row_elems, int64_t x_row_stride, uint8_t* codes,
                      int64_t code_row_stride, float* scales, int64_t scale_stride, void* stream) {
  if (!x || !codes || !scales) return DSA_ERR_ARG;
  if (x_dtype != DSA_F32 && x_dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (rows <= 0 || row_elems <= 0 || row_elems > (1 << 20) || (row_elems % 4) != 0) return DSA_ERR_SHAPE;
  if (x_row_stride < row_elems || code_row_stride < row_elems || scale_stride < 1) return DSA_ERR_SHAPE;
  const size_t esize = x_dtype == DSA_F32 ? 4 : 2;
  if (!aligned(x, 4 * esize) || (x_row_stride % 4) != 0) return DSA_ERR_ALIGN;
  if (!aligned(codes, 4) || (code_row_stride % 4) != 0 || !aligned(scales, 4)) return DSA_ERR_ALIGN;
  const hipError_t e = dsa::launch_quantize_e4m3(x, x_dtype, rows, row_elems, x_row_stride, codes, code_row_stride,
                                                 scales, scale_stride, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

int dsa_linear_bf16(const void* x, int64_t x_row_stride, const void* w, int64_t w_row_stride, int M, int N, int K,
                    float* y, int64_t y_row_stride, void* stream) {
  if (!x || !w || !y) return DSA_ERR_ARG;
  if (M <= 0 || N <= 0 || K <= 0 || (K % 64) != 0) return DSA_ERR_SHAPE;
  if (x_row_stride < K || w_row_stride < K || y_row_stride < N) return DSA_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(w, 16) || (x_row_stride % 8) != 0 || (w_row_stride % 8) != 0) return DSA_ERR_ALIGN;
  if (!aligned(y, 4)) return DSA_ERR_ALIGN;
  const hipError_t e = dsa::launch_linear_bf16(x, x_row_stride, w, w_row_stride, M, N, K, y, y_row_stride,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

int dsa_attn_probs(const dsa_attn_in* in, const float* lse, int B, int Lq, int Lk, const int32_t* idx,
                   int64_t idx_q_stride, int k, float alpha, float* P, void* stream) {
  if (!in || !lse || !idx || !P || !in->q || !in->k) return DSA_ERR_ARG;
  if (in->dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (B <= 0 || Lq <= 0 || Lk <= 0 || k <= 0) return DSA_ERR_SHAPE;
  if (in->Hkv != 1 || in->Dqk != 576 || (in->H != 16 && in->H != 32)) return DSA_ERR_SHAPE;
  if (in->k_row_stride < 576 || idx_q_stride < 0 || (idx_q_stride != 0 && idx_q_stride < k)) return DSA_ERR_SHAPE;
  if (!aligned(in->q, 16) || !aligned(in->k, 16) || (in->k_row_stride % 8) != 0) return DSA_ERR_ALIGN;
  if (!aligned(lse, 4) || !aligned(idx, 4) || !aligned(P, 4)) return DSA_ERR_ALIGN;
  dsa::AttnProbsArgs a{in->q, in->k, in->k_row_stride, lse, idx, idx_q_stride, P, in->sm_scale, alpha,
                       B, Lq, Lk, in->H, k};
  return dsa::launch_attn_probs(a, static_cast<hipStream_t>(stream)) == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

int dsa_indexer_kl_backward(const dsa_indexer_in* in, int B, int Lq, int Lk, const int32_t* idx, int k,
                            const float* pbar, float* loss, float* dq, float* dw, float* dk, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!in || !in->q || !in->k || !in->w || !idx || !pbar || !loss || !dq || !dw || !dk) return DSA_ERR_ARG;
  if (in->dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (B <= 0 || Lq <= 0 || Lk <= 0 || k <= 0 || k > dsa::kMaxKlK) return DSA_ERR_SHAPE;
  if (in->d_I != 128 || in->H_I <= 0 || in->H_I > 64 || (in->H_I % 16) != 0) return DSA_ERR_SHAPE;
  if (!aligned(in->q, 16) || !aligned(in->k, 16) || !aligned(in->w, 4)) return DSA_ERR_ALIGN;
  if (!aligned(idx, 4) || !aligned(pbar, 4) || !aligned(loss, 4) || !aligned(dq, 4) || !aligned(dw, 4) ||
      !aligned(dk, 4))
    return DSA_ERR_ALIGN;
  if (!ws || ws_bytes < dsa::indexer_kl_ws(B, Lk)) return DSA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return DSA_ERR_ALIGN;
  dsa::IndexerKlArgs a{in->q, in->k, in->w, idx, pbar, loss, dq, dw, dk,
                       static_cast<unsigned long long*>(ws), B, Lq, Lk, in->H_I, k};
  return dsa::launch_indexer_kl(a, static_cast<hipStream_t>(stream)) == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

int dsa_layer_schedule(int n_layers, int freq, int offset, const char* pattern, int32_t* anchor_out) {
  if (n_layers < 0 || !anchor_out) return DSA_ERR_ARG;
  int n_full = 0, last_full = -1;
  for (int l = 0; l < n_layers; ++l) {
    bool full;
    if (pattern) {
      if (pattern[l] == 'F') full = true;
      else if (pattern[l] == 'S') full = false;
      else return DSA_ERR_ARG;              // also a pattern shorter than n_layers
    } else {
      if (freq < 1 || offset < 0) return DSA_ERR_ARG;
      full = l < offset || (l - offset) % freq == 0;
    }
    if (full) {
      last_full = l;
      ++n_full;
    } else if (last_full < 0) {
      return DSA_ERR_ARG;                   // a Shared layer needs a Full layer before it
    }
    anchor_out[l] = last_full;
  }
  if (pattern && n_layers >= 0 && pattern[n_layers] != '\0') return DSA_ERR_ARG;
  return n_full;
}

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_ARG: return "DSA_ERR_ARG: null pointer, non-positive size or k out of range";
    case DSA_ERR_DTYPE: return "DSA_ERR_DTYPE: dtype not supported for this operation";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE: head count, head dim or stride combination not supported";
    case DSA_ERR_ALIGN: return "DSA_ERR_ALIGN: pointer or stride not aligned as required";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: a HIP call or kernel launch failed";
    default: return "unknown dsa_status";
  }
}

}  // extern "C"
