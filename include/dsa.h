/*
 * dsa.h -- C ABI of libdsa.so: DeepSeek-Sparse-Attention token selection with
 * IndexShare cross-layer index reuse, hand-written HIP kernels for gfx950 (MI355X).
 *
 * The operations follow the statement of the problem on these pages:
 *  [A] GLM-5.2 技术报告速览：IndexShare 与 critic-based PPO (mloasisblog), section
 *      "IndexShare": lightning-indexer score I[t,s] = sum_j w[t,j] ReLU(q^I[t,j] . k^I[s])
 *      over causal s <= t, then top-k (k = 2048) position IDs; groups of 4 layers with
 *      1 Full layer (runs the indexer) and 3 Shared layers (inherit its index set).
 *  [B] GLM 5.2: Built for Long Horizon Tasks (papers.chlience.com), section 5.2 (FSSS
 *      pattern; Shared layers read their own KV cache at the shared positions) and the
 *      discussion section "DSA 与 IndexShare 的组合数据流" (sparse core attention reads
 *      the selected positions' K/V of its own layer and recomputes score, softmax and
 *      value aggregation; only top-k position IDs cross layers; MLA decode uses the
 *      576-d latent: 512-d compressed KV + 64-d RoPE key).
 *  [C] GLM-5 technical report (Chinese translation), section 3.2 "Reasoning RL",
 *      paragraph "DSA RL 要点": the top-k operator must be deterministic.
 *
 * Conventions (all entry points):
 *  - Every pointer argument is DEVICE memory owned by the caller, except the struct
 *    pointers (dsa_indexer_in*, dsa_attn_in*), which are host memory read during the
 *    call only.  The library allocates no device memory and keeps no pointer after
 *    the call returns.
 *  - stream is a hipStream_t passed as void* (NULL = the default stream).  Calls only
 *    enqueue work on it; none synchronises the host.
 *  - Arguments are validated before anything is enqueued.  A negative return value
 *    (dsa_status) means nothing was enqueued.  DSA_ERR_HIP means a HIP launch error
 *    (work enqueued before the failing launch may have run).  No C++ exception crosses
 *    the ABI.  Entry points are reentrant and hold no mutable global state.
 *  - Layout: tensors are dense, row-major, innermost dimension last.  A query i of a
 *    call with Lq queries and Lk keys sits at position p_i = Lk - Lq + i and sees the
 *    keys s <= p_i (causality of [A]).
 *  - Index sets (top-k) are int32 position IDs s in [0, Lk), listed in ascending order;
 *    a row with fewer than k causal keys lists all of them followed by -1 padding; ties
 *    in score go to the lower position (reading of [C]'s determinism requirement).
 *  - FP8 operands are OCP E4M3 ("e4m3fn") codes with one fp32 scale per token; the
 *    dequantised value is code * scale.  Scales must be > 0 (the kernels factor them
 *    out of the ReLU, which is exact only for positive scales).
 *  - Scores must be finite; NaN or infinite scores make the selected set unspecified.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_ARG = -1,        /* null pointer, non-positive size, k out of range        */
  DSA_ERR_DTYPE = -2,      /* dtype not supported for this operation                  */
  DSA_ERR_SHAPE = -3,      /* head count / head dim / stride combination unsupported  */
  DSA_ERR_ALIGN = -4,      /* a pointer or stride is not aligned as required          */
  DSA_ERR_WORKSPACE = -5,  /* workspace missing or smaller than dsa_workspace_size()  */
  DSA_ERR_HIP = -6         /* a HIP call or kernel launch failed                      */
} dsa_status;

typedef enum { DSA_F32 = 0, DSA_BF16 = 1, DSA_FP8_E4M3 = 2 } dsa_dtype;

/* Operations that take a workspace (argument `op` of dsa_workspace_size). */
typedef enum {
  DSA_OP_TOPK = 0,
  DSA_OP_INDEXER_TOPK = 1,
  DSA_OP_SPARSE_ATTN = 2,
  DSA_OP_LAYER_GROUP = 3,
  DSA_OP_INDEXER_KL = 4
} dsa_op;

/*
 * Indexer operands of one Full layer ([A], indexer-score equation; [B] the indexer has
 * its own light W_Q^I / W_K^I projections and a per-layer index-key cache).
 *   q       [B, Lq, H_I, d_I]  dtype    query heads q^I
 *   q_scale [B, Lq] fp32                per-token scale (DSA_FP8_E4M3 only, else NULL)
 *   k       [B, Lk, d_I]       dtype    index-key cache k^I
 *   k_scale [B, Lk] fp32                per-token scale (DSA_FP8_E4M3 only, else NULL)
 *   w       [B, Lq, H_I] fp32           per-head gating weights w^I (any sign)
 * Supported: DSA_F32 with H_I <= 64 and H_I * d_I <= 8192 (reference-size path);
 *            DSA_BF16 / DSA_FP8_E4M3 with H_I in {16, 32, 48, 64} and d_I == 128.
 * q and k must be 16-byte aligned.
 */
typedef struct {
  const void* q;
  const float* q_scale;
  const void* k;
  const float* k_scale;
  const float* w;
  int32_t H_I;
  int32_t d_I;
  int32_t dtype; /* dsa_dtype */
} dsa_indexer_in;

/*
 * Operands of one layer's sparse core attention ([B], combined data-flow section).
 *   q    [B, Lq, H, Dqk]                       query heads (MLA: already absorbed, Dqk=576)
 *   k    [B, Lk, k_row_stride] elements        key rows: head g at offset g*Dqk
 *   v    [B, Lk, v_row_stride] elements        value rows: head g at offset g*Dv
 *                                              (MLA: v == k, Dv = 512 = the c_kv part)
 *   out  [B, Lq, H, Dv]                        written, dtype out_dtype (DSA_F32, or the
 *                                              input dtype; DSA_F32 keeps the fp32 result)
 *   lse  [B, Lq, H] fp32 or NULL               natural-log sum of exp(scaled logits);
 *                                              -inf for a query with no selected key
 * Query head h reads KV head h / (H / Hkv).  sm_scale multiplies q.k before softmax.
 * Supported: DSA_BF16 MLA latent form: H % 16 == 0, 16 <= H <= 64, Hkv == 1,
 *            Dqk == 576, Dv == 512, v == k with v_row_stride == k_row_stride (the value
 *            is the first 512 dims of the latent row), k_row_stride a multiple of 8
 *            elements >= 576, q/k/out 16-byte aligned;
 *            DSA_F32 with Dqk, Dv <= 256, H % Hkv == 0, k <= 8192 (reference-size path;
 *            k and v may be separate, k_row_stride >= Hkv*Dqk, v_row_stride >= Hkv*Dv).
 */
typedef struct {
  const void* q;
  const void* k;
  int64_t k_row_stride;
  const void* v;
  int64_t v_row_stride;
  void* out;
  float* lse;
  int32_t H;
  int32_t Hkv;
  int32_t Dqk;
  int32_t Dv;
  float sm_scale;
  int32_t dtype;     /* dsa_dtype of q, k, v */
  int32_t out_dtype; /* dsa_dtype of out: DSA_F32 or equal to dtype */
} dsa_attn_in;

/*
 * Bytes of device workspace needed by `op` (a dsa_op) for these sizes; 0 if none.
 * dtype is the indexer dtype for DSA_OP_INDEXER_TOPK / DSA_OP_LAYER_GROUP and the
 * attention dtype for DSA_OP_SPARSE_ATTN and DSA_BF16 for DSA_OP_INDEXER_KL (B and Lk are
 * the indexer's, Lq and k its query rows and index-row length); `heads` is the attention head count H for
 * DSA_OP_SPARSE_ATTN and DSA_OP_LAYER_GROUP (0 elsewhere).  For DSA_OP_TOPK the rows
 * are B * Lq rows of Lk scores (the optional workspace of dsa_topk).  The value covers both
 * idx_q_stride conventions of dsa_sparse_attn.  Pure host arithmetic, no device call;
 * returns 0 for invalid arguments (the entry point then reports them).
 */
size_t dsa_workspace_size(int op, int dtype, int B, int Lq, int Lk, int k, int heads);

/*
 * Materialised indexer scores ([A], indexer-score equation; ReLU and the head-weighted
 * sum are fused after the dot products):
 *   scores[b, i, s] = sum_j w[b,i,j] * ReLU(q[b,i,j,:] . k[b,s,:])   for s <= p_i,
 *   scores[b, i, s] = -inf                                           for s >  p_i.
 * scores: [B, Lq, Lk] fp32, written completely.  Used for short query counts (decode)
 * and for testing; the prefill path uses dsa_indexer_topk, which never writes the
 * Lq x Lk matrix.
 */
int dsa_indexer_scores(const dsa_indexer_in* in, int B, int Lq, int Lk, float* scores,
                       void* stream);

/*
 * Deterministic top-k over materialised rows ([A] top-k; [C] determinism):
 * row r holds n fp32 scores at scores + r * row_stride; only the first n_valid[r]
 * entries are candidates (n_valid == NULL means n for every row).  Writes idx[r, 0..k)
 * (ascending positions, -1 padding, ties to the lower position) and, if vals != NULL,
 * vals[r, j] = score of idx[r, j] (-inf for padding).  Requires 1 <= k <= 65536,
 * n >= 1, row_stride >= n.  The workspace is optional: with ws == NULL one workgroup
 * handles each row; with ws of at least dsa_workspace_size(DSA_OP_TOPK, 0, 1, rows, n,
 * k, 0) bytes (256-byte aligned), few long rows are split over several workgroups.
 * Both give the same result.
 */
int dsa_topk(const float* scores, int64_t row_stride, int rows, int n,
             const int32_t* n_valid, int k, int32_t* idx, float* vals, void* ws,
             size_t ws_bytes, void* stream);

/*
 * Fused indexer + top-k ([A]; the score tiles are filtered against a running per-query
 * threshold as they are produced, so the Lq x Lk score matrix is never written):
 * idx[b, i, 0..k) = top-k positions of scores[b, i, :] as defined by dsa_indexer_scores
 * and dsa_topk.  Requires 1 <= k <= 4096.  For DSA_F32 the scores of each query row are
 * written to the workspace and selected by the dsa_topk kernel.  For fewer than 16 queries
 * per sequence (decode), each chunk of keys keeps its scores on chip and writes only its
 * own top-k candidates to the workspace, from which each row is selected exactly.
 * Otherwise the fused streaming kernel runs.  The score matrix is never written.
 * ws: dsa_workspace_size(DSA_OP_INDEXER_TOPK, in->dtype, B, Lq, Lk, k, 0) bytes.
 */
int dsa_indexer_topk(const dsa_indexer_in* in, int B, int Lq, int Lk, int k,
                     int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_indexer_topk for a decode batch whose sequences hold different numbers of keys
 * (the causal rule of [A] "IndexShare" applied to each sequence on its own: a sequence
 * with n cached keys sees keys [0, n), and its query i of Lq sits at position n - Lq + i).
 * seq_lens: device int32 [B], caller-owned, n_b = seq_lens[b] clamped to [0, Lk_max].
 * k^I and k_scale are [B, Lk_max, d_I] / [B, Lk_max] caches of which sequence b uses the
 * first n_b rows (the rest are never read); q^I, q_scale and w are as in dsa_indexer_topk.
 * idx[b, i] is what dsa_indexer_topk returns for sequence b alone with Lk = n_b: its
 * top-k positions in ascending order, padded with -1 (all -1 when n_b - Lq + i < 0).
 * Requires Lq < 16, dtype DSA_BF16 or DSA_FP8_E4M3, 1 <= k <= 4096.
 * ws: dsa_workspace_size(DSA_OP_INDEXER_TOPK, in->dtype, B, Lq, Lk_max, k, 0) bytes.
 * Returns DSA_OK, DSA_ERR_ARG (null seq_lens, idx or operand), DSA_ERR_DTYPE (DSA_F32),
 * DSA_ERR_SHAPE (Lq >= 16), DSA_ERR_ALIGN, DSA_ERR_WORKSPACE or DSA_ERR_HIP.
 */
int dsa_indexer_topk_varlen(const dsa_indexer_in* in, int B, int Lq, int Lk_max, const int32_t* seq_lens,
                            int k, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_sparse_attn over an FP8 latent cache ([B] section 5.5: the training and serving
 * stack keeps the KV cache in FP8; [B] discussion section 4: FP8 KV for high-concurrency
 * decode).  in->k (== in->v, k_row_stride == v_row_stride in BYTES, a multiple of 16, at
 * least 576) holds OCP E4M3 codes, the first 576 of a row used, and kv_scale (device fp32
 * [B, Lk], caller-owned) one positive scale per row: the latent row of key s is
 * code[s] * kv_scale[s] (K all 576 dims, V the first 512).  q, out, lse, idx and every
 * other argument as in dsa_sparse_attn with in->dtype = DSA_BF16 and H = 16 or 32; the
 * result is dsa_sparse_attn's on the decoded rows.  The codes and scales are what
 * dsa_quantize_e4m3 writes for 576-value rows.
 * ws: dsa_workspace_size(DSA_OP_SPARSE_ATTN, DSA_BF16, B, Lq, Lk, k, in->H) bytes.
 * Returns as dsa_sparse_attn (DSA_ERR_ARG for a null kv_scale).
 */
int dsa_sparse_attn_kv8(const dsa_attn_in* in, const float* kv_scale, int B, int Lq, int Lk, const int32_t* idx,
                        int64_t idx_q_stride, int k, void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_indexer_topk_varlen over paged caches ([B] section 5.2: per-layer caches; the
 * serving layout stores them in fixed-size pages).  Position s of sequence b is row
 *   block_table[b * max_pages + s / page_size] * page_size + s % page_size
 * of the page pools in->k ([pool_pages * page_size, d_I]) and in->k_scale
 * ([pool_pages * page_size]); page ids outside [0, pool_pages) are clamped into it (a
 * precondition violation: the result is then unspecified but every read stays in the
 * pools).  seq_lens (device int32 [B]) as in dsa_indexer_topk_varlen, clamped to
 * [0, max_pages * page_size]; only table entries of pages below ceil(n_b / page_size) are
 * read.  page_size: a power of two, a multiple of 64, at most 2^20.  idx holds positions
 * (not pool rows) and equals dsa_indexer_topk_varlen on the same caches laid out
 * contiguously.
 * ws: dsa_workspace_size(DSA_OP_INDEXER_TOPK, in->dtype, B, Lq, max_pages * page_size, k, 0).
 * Returns DSA_OK, DSA_ERR_ARG, DSA_ERR_DTYPE (DSA_F32), DSA_ERR_SHAPE (Lq >= 16, a page size
 * or pool beyond the limits above), DSA_ERR_ALIGN, DSA_ERR_WORKSPACE or DSA_ERR_HIP.
 */
int dsa_indexer_topk_paged(const dsa_indexer_in* in, int B, int Lq, const int32_t* seq_lens,
                           const int32_t* block_table, int max_pages, int page_size, int pool_pages, int k,
                           int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Positions to pool rows for paged attention caches: rows_out[b, i, j] = the pool row of
 * position idx[b, i, j] of sequence b (block_table / page_size / pool_pages as in
 * dsa_indexer_topk_paged), or -1 where idx is -1, past max_pages * page_size, or on a page
 * id outside [0, pool_pages).  idx, rows_out: device int32 [B, Lq, k], caller-owned.  The
 * layers of a group share the block table, so one call serves all of them: dsa_sparse_attn
 * then runs with B = 1, Lq = B * Lq, Lk = pool_pages * page_size, k = the latent page pool
 * and idx = rows_out.  Returns DSA_OK, DSA_ERR_ARG, DSA_ERR_SHAPE, DSA_ERR_ALIGN or
 * DSA_ERR_HIP.
 */
int dsa_paged_rows(const int32_t* idx, int B, int Lq, int k, const int32_t* block_table, int max_pages,
                   int page_size, int pool_pages, int32_t* rows_out, void* stream);

/*
 * Sparse core attention over selected positions ([B], combined data-flow section):
 * for query (b, i), head h, with S = the entries of its idx row that lie in [0, Lk)
 * (-1 and out-of-range entries are skipped):
 *   out[b,i,h,:] = sum_{s in S} softmax_s(sm_scale * q[b,i,h,:] . K_g[s]) * V_g[s],
 *   g = h / (H / Hkv).  The idx row of (b, i) is idx + b * (idx_q_stride ? Lq *
 *   idx_q_stride : k) + i * idx_q_stride: idx_q_stride = k is one row per query,
 *   idx_q_stride = 0 makes all Lq queries of a sequence share one row (the MTP-draft
 *   reuse of the first draft step's index set, [B] section 5.3).
 * Causality is not re-applied here: attention reads exactly the listed positions, which
 * must be distinct within a row (as top-k rows are); a repeated position would be
 * weighted once per occurrence.
 * idx_q_stride must be 0 or >= k.  When few query rows are given (decode) the keys are
 * split across workgroups and combined; the partial results live in
 * ws: dsa_workspace_size(DSA_OP_SPARSE_ATTN, in->dtype, B, Lq, Lk, k, in->H) bytes.
 */
int dsa_sparse_attn(const dsa_attn_in* in, int B, int Lq, int Lk, const int32_t* idx,
                    int64_t idx_q_stride, int k, void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_sparse_attn for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc.  Same computation,
 * same kernels and the same result as dsa_sparse_attn; the partial results of keys split
 * over several workgroups (few query rows, i.e. decode) go to a buffer the library owns
 * instead of a caller workspace: a static device array of DSA_NOALLOC_SCRATCH_BYTES, one
 * copy on each GPU the library runs on, held until the process ends.  The call allocates
 * nothing (no hipMalloc, no allocating library routine); the caller still provides q, the
 * cache, idx, out and lse.
 * Limit: DSA_NOALLOC_SCRATCH_BYTES (40 MiB) holds the split partials of every call with at
 * most 32 heads and at most 256 query rows (B * Lq: the decode and MTP-draft shapes, which
 * need at most 32 MiB), and calls with 1024 or more query rows need none.  A call whose
 * dsa_workspace_size(DSA_OP_SPARSE_ATTN, ...) exceeds it returns DSA_ERR_WORKSPACE before
 * anything is enqueued.
 * Concurrency: every call on a GPU shares that GPU's buffer, which keeps the last call's
 * contents; calls ordered on one stream are safe, calls that overlap on one GPU (other
 * streams, other threads) race and give undefined results.  The first call on a device
 * looks up the buffer's device address with that device current (the device of `stream`).
 * Returns as dsa_sparse_attn, or DSA_ERR_HIP if that lookup fails.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (40u << 20)
int dsa_sparse_attn_noalloc(const dsa_attn_in* in, int B, int Lq, int Lk, const int32_t* idx,
                            int64_t idx_q_stride, int k, void* stream);

/*
 * One IndexShare group ([A] section "IndexShare"; [B] section 5.2): the Full layer's
 * indexer + top-k runs once (dsa_indexer_topk with `full`), writing idx_out [B, Lq, k];
 * then layers[0..n_layers) each run dsa_sparse_attn with that same idx (layer 0 is the
 * Full layer's own attention, layers 1.. are the Shared layers).  n_layers = 0 is
 * dsa_indexer_topk alone.  The all-Full comparator is n_layers = 1 called once per layer
 * with each layer's own indexer operands.
 * All layers must share dtype, H, Dqk and Dv.  The attention runs with idx_q_stride = k.
 * ws: dsa_workspace_size(DSA_OP_LAYER_GROUP, full->dtype, B, Lq, Lk, k, layers[0].H)
 * bytes (covers the indexer and the attention, which run one after the other).
 */
int dsa_layer_group(const dsa_indexer_in* full, const dsa_attn_in* layers, int n_layers,
                    int B, int Lq, int Lk, int k, int32_t* idx_out, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * Per-token E4M3 quantization of indexer operands, the step before the path ([A]
 * "IndexShare": the indexer is kept FP8-friendly; [B] section 5.2: its own light
 * projections and a per-layer index-key cache).  Row r holds row_elems values (one
 * token: H_I * d_I for q^I, d_I for k^I) at x + r * x_row_stride elements, fp32 or bf16
 * (x_dtype).  It writes
 *   scales[r * scale_stride] = amax_r / 448 (1 for an all-zero row), single precision;
 *   codes[r * code_row_stride + e] = OCP E4M3 code of x[r][e] / scale, round to nearest
 *   even, sign kept.
 * These are exactly the codes and scales the indexer entry points consume.  Strided
 * destinations let a decode step append each sequence's new k^I row to its cache slot:
 * codes = k_cache + p * d_I, code_row_stride = Lk_max * d_I, scales = k_scale_cache + p,
 * scale_stride = Lk_max.
 * All pointers are caller-owned device memory.  row_elems must be a multiple of 4 (at most
 * 2^20), x 16-byte (fp32) or 8-byte (bf16) aligned with x_row_stride a multiple of 4,
 * codes and scales 4-byte aligned with code_row_stride a multiple of 4.  NaN or infinite
 * inputs are a precondition violation.  Returns DSA_OK, DSA_ERR_ARG, DSA_ERR_DTYPE,
 * DSA_ERR_SHAPE, DSA_ERR_ALIGN or DSA_ERR_HIP.
 */
int dsa_quantize_e4m3(const void* x, int x_dtype, int rows, int row_elems, int64_t x_row_stride, uint8_t* codes,
                      int64_t code_row_stride, float* scales, int64_t scale_stride, void* stream);

/*
 * bf16 linear map for the indexer's projections, the step before dsa_quantize_e4m3 ([B]
 * discussion section "DSA 与 IndexShare 的组合数据流": the indexer keeps its own light
 * projections W_Q^I, W_K^I beside the MLA path; [A] "IndexShare": per-head gating weights
 * w^I).  The pages give neither the projections' input nor their widths; they are read as
 * linear maps of the layer's hidden state h.  For the hidden states h of M
 * tokens it computes q^I = h W_Q^I (N = H_I * d_I), k^I = h W_K^I (N = d_I) and
 * w = h W_w (N = H_I), one call per weight:
 *   y[m * y_row_stride + n] = sum_k x[m * x_row_stride + k] * w[n * w_row_stride + k],
 * i.e. x [M, K] and w [N, K] are row-major bf16 (w in the layout of a linear layer's
 * weight) and y [M, N] is fp32, each output one dot product accumulated in fp32 by the
 * bf16 matrix cores (the products are exact in fp32; the sum order is the kernel's).
 * All pointers are caller-owned device memory.  K must be a positive multiple of 64;
 * x_row_stride, w_row_stride >= K and multiples of 8, y_row_stride >= N; x and w 16-byte
 * aligned, y 4-byte aligned.  Returns DSA_OK, DSA_ERR_ARG (null pointer), DSA_ERR_SHAPE,
 * DSA_ERR_ALIGN or DSA_ERR_HIP.
 */
int dsa_linear_bf16(const void* x, int64_t x_row_stride, const void* w, int64_t w_row_stride, int M, int N, int K,
                    float* y, int64_t y_row_stride, void* stream);

/*
 * Training of the kept indexer ([A] "IndexShare": reusing one index set across a group
 * of layers loses accuracy when each indexer was trained for its own layer only, so the
 * kept indexer is fit by KL to the centroid pbar_t = 1/(m+1) sum_j p_t^(l+j) of the
 * head-averaged attention distributions of the m + 1 layers it serves).  Read in the
 * sparse form: both distributions live on the query's index row S_t.
 *
 * dsa_attn_probs: one layer's head-averaged distribution on S_t, accumulated with weight
 * alpha (1/(m+1) to build the centroid over a group):
 *   P[r, i] += alpha / H * sum_h exp(sm_scale * q[r, h] . K[S_r[i]] - lse[r, h])
 * for idx entries S_r[i] in [0, Lk) (other entries are left unchanged).  in is the
 * layer's dsa_attn_in as given to dsa_sparse_attn (MLA: Hkv = 1, Dqk = 576, bf16, H = 16
 * or 32; K is the whole latent row); lse [B, Lq, H] is what dsa_sparse_attn wrote for the
 * same idx (natural-log sum of exp(sm_scale q . K) over the row); the idx row of (b, i) is
 * that of dsa_sparse_attn, idx + b * (idx_q_stride ? Lq * idx_q_stride : k) + i *
 * idx_q_stride (idx_q_stride = k: one row per query; 0: the Lq queries of a sequence share
 * one row), k entries; P [B, Lq, k] fp32, caller-owned.
 * Returns DSA_OK, DSA_ERR_ARG, DSA_ERR_DTYPE, DSA_ERR_SHAPE, DSA_ERR_ALIGN or DSA_ERR_HIP.
 */
int dsa_attn_probs(const dsa_attn_in* in, const float* lse, int B, int Lq, int Lk, const int32_t* idx,
                   int64_t idx_q_stride, int k, float alpha, float* P, void* stream);

/*
 * dsa_indexer_kl_backward: loss and gradients of sum_r KL(pbar_r || pi_r), pi_r the
 * softmax over S_r of the indexer scores I[r, s] = sum_j w[r, j] ReLU(q[r, j] . k[s])
 * (the indexer-score equation of [A]), with g = pi - pbar:
 *   loss[r] = sum_{s in S_r, pbar > 0} pbar (log pbar - log pi)
 *   dw[r, j] = sum_s g[s] ReLU(x),  dq[r, j, :] = sum_s g[s] w[r, j] [x > 0] k[s]
 *   dk[s, :] += sum_r sum_j g[s] w[r, j] [x > 0] q[r, j]      (x = q[r, j] . k[s])
 * in: bf16 q^I [B, Lq, H_I, 128] and k^I [B, Lk, 128], fp32 w [B, Lq, H_I] (H_I a multiple
 * of 16, at most 64; d_I = 128); idx [B, Lq, k] (entries outside [0, Lk) are not in S_r;
 * positions within a row must be distinct), k <= 2048; pbar [B, Lq, k] aligned with idx
 * (mass only on entries in S_r).  Outputs fp32, caller-owned: loss [B, Lq], dq, dw, and
 * dk [B, Lk, 128], to which this call's dk is ADDED (zero it for a fresh result).  dk is deterministic:
 * each contribution is rounded to a multiple of 2^-30 and the contributions of a key are
 * summed as 64-bit integers in the workspace, so the sum does not depend on the order in
 * which the rows add them (each key's partial sums must stay below 2^33 in magnitude);
 * the sum is then converted and added to dk.  The contractions run on the bf16 matrix
 * cores with fp32 accumulation; the coefficients g w [x > 0] enter them rounded to bf16.
 * ws: dsa_workspace_size(DSA_OP_INDEXER_KL, DSA_BF16, B, Lq, Lk, k, 0) bytes (256-byte
 * aligned).  Returns DSA_OK, DSA_ERR_ARG, DSA_ERR_DTYPE, DSA_ERR_SHAPE, DSA_ERR_ALIGN,
 * DSA_ERR_WORKSPACE or DSA_ERR_HIP.
 */
int dsa_indexer_kl_backward(const dsa_indexer_in* in, int B, int Lq, int Lk, const int32_t* idx, int k,
                            const float* pbar, float* loss, float* dq, float* dw, float* dk, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * Layer schedule of an IndexShare stack ([B] section 5.2: the released configuration
 * sets index_topk_freq = 4, index_skip_topk_offset = 3 and no explicit pattern, and
 * after the offset the indexer types repeat full, shared, shared, shared; [A] section
 * "IndexShare": a Shared layer uses the index set of the nearest Full layer before it).
 * Host only: no device memory, no stream, nothing enqueued.
 *   pattern == NULL: layer l is Full when l < offset or (l - offset) % freq == 0
 *     (freq >= 1, offset >= 0; the pages leave the meaning of the offset open, this reads
 *     it as that many leading Full layers before the periodic part);
 *   pattern != NULL: a string of exactly n_layers characters 'F' / 'S' (the explicit
 *     per-layer pattern); freq and offset are ignored.
 * anchor_out [n_layers] (host memory, caller-owned) receives, for every layer, the index
 * of the Full layer whose idx it attends with (its own index for a Full layer).
 * Returns the number of Full layers (>= 0), or DSA_ERR_ARG for n_layers < 0, a null
 * anchor_out, freq < 1 or offset < 0 without a pattern, a pattern of another length or
 * with other characters, or a Shared layer with no Full layer before it (anchor_out is
 * then partly written).
 */
int dsa_layer_schedule(int n_layers, int freq, int offset, const char* pattern, int32_t* anchor_out);

/* Static string naming a status code. */
const char* dsa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
