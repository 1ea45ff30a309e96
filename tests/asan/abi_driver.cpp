// Host-side driver of the C ABI's argument validation, built with AddressSanitizer over a
// host-only compile of the library sources (no device code, no GPU).  Every call below is
// rejected before any HIP call, so the driver exercises exactly the validation layer; the
// host-only entry points (workspace sizes, layer schedule, status strings) run in full.
// Exit status 0 when every call returns the expected status.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>

#include "dsa.h"

static int failures = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const long long got_ = (long long)(call);                                           \
    if (got_ != (long long)(want)) {                                                    \
      fprintf(stderr, "line %d: %s returned %lld, expected %lld\n", __LINE__, #call,    \
              got_, (long long)(want));                                                  \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

static dsa_indexer_in ind(int dtype, int H_I = 64, int d_I = 128, uintptr_t q = 0x1000, uintptr_t qs = 0x6000,
                          uintptr_t ks = 0x7000) {
  dsa_indexer_in s;
  memset(&s, 0, sizeof(s));
  s.q = P(q);
  s.k = P(0x2000);
  s.w = static_cast<const float*>(P(0x3000));
  s.q_scale = dtype == DSA_FP8_E4M3 ? static_cast<const float*>(P(qs)) : nullptr;
  s.k_scale = dtype == DSA_FP8_E4M3 ? static_cast<const float*>(P(ks)) : nullptr;
  s.H_I = H_I;
  s.d_I = d_I;
  s.dtype = dtype;
  return s;
}

static dsa_attn_in att(int H = 32, uintptr_t q = 0x1000, int64_t stride = 576, int dtype = DSA_BF16) {
  dsa_attn_in a;
  memset(&a, 0, sizeof(a));
  a.q = P(q);
  a.k = a.v = P(0x2000);
  a.k_row_stride = a.v_row_stride = stride;
  a.out = P(0x3000);
  a.H = H;
  a.Hkv = 1;
  a.Dqk = 576;
  a.Dv = 512;
  a.sm_scale = 0.04f;
  a.dtype = dtype;
  a.out_dtype = dtype;
  return a;
}

int main() {
  const int32_t* idx = static_cast<const int32_t*>(P(0x5000));
  int32_t* idx_out = static_cast<int32_t*>(P(0x5000));
  void* ws = P(0x100000);
  const size_t big = (size_t)1 << 40;

  // workspace sizes: pure host arithmetic, 0 for invalid arguments, no overflow wrap
  EXPECT(dsa_workspace_size(DSA_OP_TOPK, DSA_F32, 1, 16, 1000, 64, 0), 0);
  EXPECT(dsa_workspace_size(DSA_OP_INDEXER_TOPK, 7, 1, 16, 16, 4, 0), 0);
  EXPECT(dsa_workspace_size(DSA_OP_INDEXER_TOPK, DSA_BF16, 1, 32, 16, 4, 0), 0);
  EXPECT(dsa_workspace_size(DSA_OP_INDEXER_TOPK, DSA_BF16, -1, 32, 64, 4, 0), 0);
  EXPECT(dsa_workspace_size(99, DSA_BF16, 1, 32, 64, 4, 0), 0);
  EXPECT(dsa_workspace_size(DSA_OP_SPARSE_ATTN, DSA_BF16, 64, 1, 200001, 2048, 32) > 0, 1);
  EXPECT(dsa_workspace_size(DSA_OP_INDEXER_TOPK, DSA_FP8_E4M3, 64, 1, 200001, 2048, 0) >= (size_t)64 * 200001 * 8, 1);
  EXPECT(dsa_workspace_size(DSA_OP_INDEXER_TOPK, DSA_FP8_E4M3, 1, 131072, 131072, 2048, 0) > 0, 1);

  // indexer + top-k
  dsa_indexer_in b = ind(DSA_BF16);
  EXPECT(dsa_indexer_topk(nullptr, 1, 64, 64, 16, idx_out, ws, big, nullptr), DSA_ERR_ARG);
  dsa_indexer_in noq = b;
  noq.q = nullptr;
  EXPECT(dsa_indexer_topk(&noq, 1, 64, 64, 16, idx_out, ws, big, nullptr), DSA_ERR_ARG);
  dsa_indexer_in bad_dt = ind(9);
  EXPECT(dsa_indexer_topk(&bad_dt, 1, 64, 64, 16, idx_out, ws, big, nullptr), DSA_ERR_DTYPE);
  dsa_indexer_in bad_h = ind(DSA_BF16, 40);
  EXPECT(dsa_indexer_topk(&bad_h, 1, 64, 64, 16, idx_out, ws, big, nullptr), DSA_ERR_SHAPE);
  dsa_indexer_in bad_d = ind(DSA_BF16, 64, 64);
  EXPECT(dsa_indexer_topk(&bad_d, 1, 64, 64, 16, idx_out, ws, big, nullptr), DSA_ERR_SHAPE);
  dsa_indexer_in mis = ind(DSA_BF16, 64, 128, 0x1004);
  EXPECT(dsa_indexer_topk(&mis, 1, 64, 64, 16, idx_out, ws, big, nullptr), DSA_ERR_ALIGN);
  dsa_indexer_in fp8_noscale = ind(DSA_FP8_E4M3, 64, 128, 0x1000, 0, 0);
  EXPECT(dsa_indexer_topk(&fp8_noscale, 1, 64, 64, 16, idx_out, ws, big, nullptr), DSA_ERR_ARG);
  EXPECT(dsa_indexer_topk(&b, 1, 65, 64, 16, idx_out, ws, big, nullptr), DSA_ERR_ARG);
  EXPECT(dsa_indexer_topk(&b, 1, 64, 64, 0, idx_out, ws, big, nullptr), DSA_ERR_ARG);
  EXPECT(dsa_indexer_topk(&b, 1, 64, 64, 5000, idx_out, ws, big, nullptr), DSA_ERR_ARG);
  EXPECT(dsa_indexer_topk(&b, 1, 64, 64, 16, idx_out, nullptr, big, nullptr), DSA_ERR_WORKSPACE);
  EXPECT(dsa_indexer_topk(&b, 1, 64, 64, 16, idx_out, ws, 16, nullptr), DSA_ERR_WORKSPACE);
  EXPECT(dsa_indexer_scores(&b, 1, 4, 4, nullptr, nullptr), DSA_ERR_ARG);
  dsa_indexer_in f8 = ind(DSA_FP8_E4M3);
  const int32_t* lens = static_cast<const int32_t*>(P(0x5800));
  EXPECT(dsa_indexer_topk_varlen(&f8, 2, 1, 64, nullptr, 16, idx_out, ws, big, nullptr), DSA_ERR_ARG);
  EXPECT(dsa_indexer_topk_varlen(&f8, 2, 16, 64, lens, 16, idx_out, ws, big, nullptr), DSA_ERR_SHAPE);
  EXPECT(dsa_indexer_topk_varlen(&f8, 2, 1, 64, lens, 16, idx_out, ws, 16, nullptr), DSA_ERR_WORKSPACE);
  const int32_t* table = static_cast<const int32_t*>(P(0x8000));
  for (int page : {32, 96, 100, 1 << 21})
    EXPECT(dsa_indexer_topk_paged(&f8, 2, 1, lens, table, 4, page, 16, 16, idx_out, ws, big, nullptr), DSA_ERR_SHAPE);
  EXPECT(dsa_indexer_topk_paged(&f8, 2, 1, lens, nullptr, 4, 64, 16, 16, idx_out, ws, big, nullptr), DSA_ERR_ARG);
  EXPECT(dsa_paged_rows(idx, 1, 1, 8, table, 4, 48, 16, idx_out, nullptr), DSA_ERR_SHAPE);
  EXPECT(dsa_paged_rows(nullptr, 1, 1, 8, table, 4, 64, 16, idx_out, nullptr), DSA_ERR_ARG);

  // top-k of materialised rows
  const float* sc = static_cast<const float*>(P(0x1000));
  EXPECT(dsa_topk(nullptr, 8, 1, 8, nullptr, 4, idx_out, nullptr, nullptr, 0, nullptr), DSA_ERR_ARG);
  EXPECT(dsa_topk(sc, 4, 1, 8, nullptr, 4, idx_out, nullptr, nullptr, 0, nullptr), DSA_ERR_ARG);
  EXPECT(dsa_topk(sc, 8, 1, 8, nullptr, 0, idx_out, nullptr, nullptr, 0, nullptr), DSA_ERR_ARG);
  EXPECT(dsa_topk(sc, 8, 1, 8, nullptr, 65537, idx_out, nullptr, nullptr, 0, nullptr), DSA_ERR_ARG);
  EXPECT(dsa_topk(static_cast<const float*>(P(0x1002)), 8, 1, 8, nullptr, 4, idx_out, nullptr, nullptr, 0, nullptr),
         DSA_ERR_ALIGN);

  // sparse attention, its FP8-latent and allocation-free forms
  dsa_attn_in a = att();
  EXPECT(dsa_sparse_attn(&a, 1, 4, 64, nullptr, 16, 16, ws, big, nullptr), DSA_ERR_ARG);
  EXPECT(dsa_sparse_attn(&a, 1, 4, 64, idx, 8, 16, ws, big, nullptr), DSA_ERR_ARG);
  dsa_attn_in h40 = att(40);
  EXPECT(dsa_sparse_attn(&h40, 1, 4, 64, idx, 16, 16, ws, big, nullptr), DSA_ERR_SHAPE);
  dsa_attn_in st = att(32, 0x1000, 580);
  EXPECT(dsa_sparse_attn(&st, 1, 4, 64, idx, 16, 16, ws, big, nullptr), DSA_ERR_ALIGN);
  dsa_attn_in fp8a = att(32, 0x1000, 576, DSA_FP8_E4M3);
  EXPECT(dsa_sparse_attn(&fp8a, 1, 4, 64, idx, 16, 16, ws, big, nullptr), DSA_ERR_DTYPE);
  EXPECT(dsa_sparse_attn(&a, 2, 1, 5000, idx, 2048, 2048, nullptr, 0, nullptr), DSA_ERR_WORKSPACE);
  const float* kvs = static_cast<const float*>(P(0x7000));
  EXPECT(dsa_sparse_attn_kv8(&a, nullptr, 1, 4, 64, idx, 16, 16, ws, big, nullptr), DSA_ERR_ARG);
  dsa_attn_in h48 = att(48);
  EXPECT(dsa_sparse_attn_kv8(&h48, kvs, 1, 4, 64, idx, 16, 16, ws, big, nullptr), DSA_ERR_SHAPE);
  EXPECT(dsa_sparse_attn_noalloc(&a, 1, 4, 64, nullptr, 16, 16, nullptr), DSA_ERR_ARG);
  EXPECT(dsa_sparse_attn_noalloc(&a, 300, 1, 1000000, idx, 2048, 2048, nullptr), DSA_ERR_WORKSPACE);

  // layer group
  dsa_attn_in layers[2] = {att(32), att(16)};
  EXPECT(dsa_layer_group(&b, layers, 2, 1, 64, 64, 16, idx_out, ws, big, nullptr), DSA_ERR_SHAPE);
  EXPECT(dsa_layer_group(&b, nullptr, 1, 1, 64, 64, 16, idx_out, ws, big, nullptr), DSA_ERR_ARG);

  // quantization, projections, objective
  EXPECT(dsa_quantize_e4m3(P(0x1000), 5, 4, 128, 128, static_cast<uint8_t*>(P(0x2000)), 128,
                           static_cast<float*>(P(0x3000)), 1, nullptr), DSA_ERR_DTYPE);
  EXPECT(dsa_quantize_e4m3(P(0x1000), DSA_F32, 4, 126, 128, static_cast<uint8_t*>(P(0x2000)), 128,
                           static_cast<float*>(P(0x3000)), 1, nullptr), DSA_ERR_SHAPE);
  EXPECT(dsa_linear_bf16(P(0x1000), 96, P(0x2000), 96, 4, 4, 96, static_cast<float*>(P(0x3000)), 4, nullptr),
         DSA_ERR_SHAPE);
  EXPECT(dsa_linear_bf16(nullptr, 64, P(0x2000), 64, 4, 4, 64, static_cast<float*>(P(0x3000)), 4, nullptr),
         DSA_ERR_ARG);
  const float* lse = static_cast<const float*>(P(0x7000));
  float* pp = static_cast<float*>(P(0x6000));
  EXPECT(dsa_attn_probs(&a, nullptr, 1, 4, 64, idx, 16, 16, 0.5f, pp, nullptr), DSA_ERR_ARG);
  EXPECT(dsa_attn_probs(&h48, lse, 1, 4, 64, idx, 16, 16, 0.5f, pp, nullptr), DSA_ERR_SHAPE);
  EXPECT(dsa_indexer_kl_backward(&b, 1, 8, 64, idx, 4096, pp, pp, pp, pp, pp, ws, big, nullptr), DSA_ERR_SHAPE);
  EXPECT(dsa_indexer_kl_backward(&f8, 1, 8, 64, idx, 64, pp, pp, pp, pp, pp, ws, big, nullptr), DSA_ERR_DTYPE);
  EXPECT(dsa_indexer_kl_backward(&b, 1, 8, 64, idx, 64, pp, pp, pp, pp, pp, nullptr, big, nullptr), DSA_ERR_WORKSPACE);
  EXPECT(dsa_workspace_size(DSA_OP_INDEXER_KL, DSA_BF16, 1, 8, 64, 64, 0), (size_t)64 * 128 * 8);
  EXPECT(dsa_workspace_size(DSA_OP_INDEXER_KL, DSA_FP8_E4M3, 1, 8, 64, 64, 0), 0);

  // layer schedule (host only, runs in full): patterns in exactly sized buffers
  int32_t anchors[80];
  EXPECT(dsa_layer_schedule(80, 4, 3, nullptr, anchors), 23);
  EXPECT(dsa_layer_schedule(80, 4, 0, nullptr, anchors), 20);
  EXPECT(anchors[79], 76);
  const char* pats[] = {"F", "FSSS", "FFFSSSFS"};
  const int fulls[] = {1, 1, 4};
  for (int i = 0; i < 3; ++i) {
    const size_t n = strlen(pats[i]);
    char* exact = static_cast<char*>(malloc(n + 1));
    memcpy(exact, pats[i], n + 1);
    EXPECT(dsa_layer_schedule((int)n, 4, 0, exact, anchors), fulls[i]);
    free(exact);
  }
  char* shorter = static_cast<char*>(malloc(3));
  memcpy(shorter, "FS", 3);
  EXPECT(dsa_layer_schedule(3, 4, 0, shorter, anchors), DSA_ERR_ARG);   // stops at the terminator
  free(shorter);
  EXPECT(dsa_layer_schedule(3, 4, 0, "SFF", anchors), DSA_ERR_ARG);
  EXPECT(dsa_layer_schedule(3, 4, 0, "FSSS", anchors), DSA_ERR_ARG);
  EXPECT(dsa_layer_schedule(3, 0, 0, nullptr, anchors), DSA_ERR_ARG);
  EXPECT(dsa_layer_schedule(-1, 4, 0, nullptr, anchors), DSA_ERR_ARG);
  EXPECT(dsa_layer_schedule(3, 4, 0, nullptr, nullptr), DSA_ERR_ARG);
  for (int code = 0; code >= -7; --code) EXPECT(strncmp(dsa_status_string(code), code == -7 ? "unknown" : "DSA_", 4), 0);

  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("abi validation: all calls returned the expected status\n");
  return 0;
}
