// Sparse core attention over selected positions (gfx950).
//
// GLM 5.2: Built for Long Horizon Tasks, discussion section "DSA 与 IndexShare 的组合数据流":
// each layer reads the K/V of the selected positions from its own cache and recomputes
// score, softmax and value aggregation on them only.  MLA latent form (GLM-5 technical
// report section 2.1; same discussion section): one 576-d latent row per key (512-d
// compressed KV + 64-d RoPE key); K is the whole row, V its first 512 dims, and the
// query heads are already absorbed to 576-d.
//
// Two MLA kernels: mla_attn32_kernel (32-key blocks, below) serves 16 and 32 heads;
// mla_attn_kernel (16-key blocks, first) serves 48 and 64 heads.
//
// mla_attn_kernel: one workgroup per (query row group, key split); a row group is the nq
// queries that share one idx row (nq = 1, or the MTP draft queries).  Each wave owns
// 16 heads of one query.  Keys are processed in blocks of 16 selected positions: the
// block's 16 latent rows (18 KB) are gathered straight into LDS with direct-to-LDS loads
// (global_load_lds_dwordx4), double-buffered so that block n+1 is in flight while block n
// is computed; the idx row is read two blocks ahead.  Per block every wave computes
//   S^T[key, head] = K . Q^T  (bf16 MFMA 16x16x32, K from LDS, Q^T held in registers),
// an online softmax per head (each lane owns one head; the running maximum is only
// raised when it grows by more than 2^8, so the O rescale is rare), and
//   O^T[dv, head] += V^T . P^T  (one 16x16x32 MFMA per 16 dims: the K=32 slots carry the
// 16 keys twice, once with bf16(p) and once with the bf16 residual p - bf16(p), so P
// enters with ~16 bits; V^T comes from the row-major LDS tile through the transposing
// LDS read ds_read_b64_tr_b16).
// LDS rows are stored with the 16-byte chunks of each group of 8 XOR-swizzled by
// (row/2) % 8, so the 16 rows read by one MFMA operand fall in distinct banks.
#include "dsa_common.hpp"
#include "dsa_launch.hpp"
#include "mla_blocks.hpp"
#include "../../include/dsa.h"

namespace dsa {

constexpr int kDmaPerBlk = kBlkBytes / 1024;    // 18 wave-wide 1 KB direct-to-LDS loads
constexpr float kRescaleGap = 8.0f;             // log2 headroom before the max is raised
constexpr float kMaxStart = 1e30f;              // initial running maximum is -kMaxStart
constexpr int kKeyBufs = 4;                     // idx ring slots (j .. j+2 in use)

__device__ __forceinline__ bf16x4 lds_read_tr16(const uint8_t* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ __forceinline__ f32x4 sp_plus(f32x4 lo_half, f32x4 hi_half) { return lo_half + hi_half; }

// LDS chunk slot of global 16-byte chunk c of block row r (an involution).
__device__ __forceinline__ int swz(int r, int c) { return (c & ~7) | ((c & 7) ^ ((r >> 1) & 7)); }

struct MlaParams {
  AttnArgs a;
  int nq;            // queries sharing one idx row
  int n_groups;      // B * Lq / nq
  int n_split;
  int blocks_per_split;
  float* part_o;     // [n_groups*nq*H][n_split][512]   (n_split > 1)
  float* part_ml;    // [n_groups*nq*H][n_split][2]
};

// NW waves per workgroup; DVS = slices of the 512 value dims per (query, head tile):
// DVS = 2 halves the output accumulators a wave holds (16 heads x 256 dims).  The two
// slices of a head tile also split the S^T reduction: each multiplies over 288 of the 576
// latent dims, the partial tiles are exchanged through LDS, and both add them in the same
// order (so both hold bitwise the same S^T).  WPE = minimum waves per SIMD the register
// allocation must allow.  SPLIT: the keys are split over blockIdx.y and the kernel writes
// unnormalised partials (o, m, l) for mla_combine_kernel instead of the output.  NB = row
// buffers: 2 keeps one block of rows in flight (more workgroups fit a CU), 3 keeps up to
// two in flight (for the few, long-latency workgroups of decode).
template <int NW, int DVS, int WPE, bool SPLIT, int NB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void mla_attn_kernel(MlaParams P) {
  constexpr int kDvPer = kMlaDv / DVS;          // value dims per wave
  constexpr int kDt = kDvPer / 16;              // 16-dim output tiles per wave
  constexpr int kQSteps = 18 / DVS;             // 32-dim QK MFMA steps per wave
  constexpr int kSlotsPerWave = (kDmaPerBlk + NW - 1) / NW;
  constexpr int kDummy = kSlotsPerWave * NW - kDmaPerBlk;   // padding slots (fixed counts)
  __shared__ __attribute__((aligned(16))) uint8_t kvs[NB][kBlkBytes + kDummy * 1024];
  __shared__ __attribute__((aligned(16))) int keyring[kKeyBufs][64];   // idx entries of blocks
  __shared__ __attribute__((aligned(16))) f32x4 xch[DVS == 2 ? 2 : 1][DVS == 2 ? NW : 1][64];  // partial S^T
  const AttnArgs& a = P.a;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int wv_id = uniform(tid >> 6);      // wave index, kept in a scalar register
  const int hpq = a.H / 16;                 // head tiles per query
  const int wpq = hpq * DVS;                // waves per query
  // XCD-aware order: consecutive workgroup ids go to different XCDs; give each XCD a
  // contiguous range of row groups (neighbouring queries share many selected rows).
  const int ng = P.n_groups;
  int grp;
  {
    const int bid = blockIdx.x, xcd = bid & 7, j = bid >> 3;
    const int per = ng >> 3, rem = ng & 7;
    grp = (xcd < rem) ? xcd * (per + 1) + j : rem * (per + 1) + (xcd - rem) * per + j;
  }
  const int split = blockIdx.y;
  const int qpl = a.Lq / P.nq;              // row groups per sequence
  const int b = grp / qpl;
  const int qi = wv_id / wpq;
  const int wr = wv_id - qi * wpq;
  const int ht = wr % hpq;                  // head tile
  const int ds = wr / hpq;                  // value-dim slice
  const int i = (grp - b * qpl) * P.nq + qi;
  const bool wave_active = wv_id < P.nq * wpq;
  const int32_t* idx_row = a.idx_q_stride
                               ? a.idx + (size_t)b * a.Lq * a.idx_q_stride + (size_t)((grp - b * qpl) * P.nq) * a.idx_q_stride
                               : a.idx + (size_t)b * a.topk;
  const int n_blk_total = (a.topk + kBlk - 1) / kBlk;
  const int blk_begin = split * P.blocks_per_split;
  const int blk_end = min(n_blk_total, blk_begin + P.blocks_per_split);
  const uint8_t* kvbase = reinterpret_cast<const uint8_t*>(a.k) + (size_t)b * a.Lk * a.k_row_stride * 2;
  const size_t row_bytes = (size_t)a.k_row_stride * 2;

  // idx entries of a block into its ring slot (lanes 0..15).  Every wave issues the same
  // load (same bytes to the same place) so that all waves count the same number of loads.
  // Positions past topk (a last partial block) are stored as -1.
  auto issue_keys = [&](int blk) {
    int* slot = &keyring[(blk - blk_begin) & (kKeyBufs - 1)][0];
    const int pos = blk * kBlk + lane;
    if (lane < kBlk) {
      if (pos < a.topk) dma_4(idx_row + pos, lds_offset(slot));
      else slot[lane] = -1;
    }
  };
  // the block's 16 latent rows into kvs[buf] (rows of invalid entries read row 0 and are
  // masked later).  Every wave issues the same number of loads; padding slots fill a dummy
  // area.  The ring entries are read first: the loads below are ordered after them.
  int dma_row[kSlotsPerWave];
  const uint8_t* dma_src[kSlotsPerWave];
#pragma unroll
  for (int u = 0; u < kSlotsPerWave; ++u) {
    const int j = wv_id + u * NW;
    const int piece = j * 64 + lane;
    const int r = min(piece / kChunks, kBlk - 1);
    const int cs = piece - (piece / kChunks) * kChunks;
    dma_row[u] = r;
    dma_src[u] = kvbase + (j < kDmaPerBlk ? 16 * swz(r, cs) : 0);
  }
  const uint32_t row_bytes32 = (uint32_t)row_bytes;
  auto issue_rows = [&](int blk, int buf) {
    const int* slot = &keyring[(blk - blk_begin) & (kKeyBufs - 1)][0];
    int key[kSlotsPerWave];
#pragma unroll
    for (int u = 0; u < kSlotsPerWave; ++u) key[u] = slot[dma_row[u]];
#pragma unroll
    for (int u = 0; u < kSlotsPerWave; ++u) {
      const uint32_t kk = (uint32_t)key[u] < (uint32_t)a.Lk ? (uint32_t)key[u] : 0u;
      dma_16(dma_src[u] + (uint64_t)kk * row_bytes32, lds_offset(&kvs[buf][(wv_id + u * NW) * 1024]));
    }
  };

  // Q^T operand: head h, dims [32 (ks + kQSteps ds) + 8 g, +8) for this wave's half
  const int h = ht * 16 + r16;
  bf16x8 qop[kQSteps];
  {
    const int qq = wave_active ? i : 0;
    const bf16x8* qrow = reinterpret_cast<const bf16x8*>(
        reinterpret_cast<const uint16_t*>(a.q) + (((size_t)b * a.Lq + qq) * a.H + (wave_active ? h : 0)) * kMlaD);
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) qop[ks] = qrow[4 * (ks + kQSteps * ds) + g];
  }
  const int partner = wv_id + (ds == 0 ? hpq : -hpq);   // same head tile, other half (DVS = 2)
  f32x4 o[kDt];
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // running maximum in log2 units of the scaled logits; finite so that exp2 of an invalid
  // (-inf) logit minus it is 0 and the first raise multiplies the empty state by 0
  float m_use = -kMaxStart, l_lane = 0.f;
  const float sl2 = a.sm_scale * kLog2e;
  // loop-invariant LDS offsets (bytes within a row buffer)
  // this wave's half starts at 32-dim step kQSteps*ds (chunk 4*kQSteps*ds; kQSteps is odd,
  // so the parity of the step index flips between the halves)
  const int ks0 = kQSteps * ds;
  const int k_off0 = r16 * kRowBytes + 16 * swz(r16, 4 * (ks0 & 1) + g) + 128 * (ks0 >> 1);
  const int k_off1 = r16 * kRowBytes + 16 * swz(r16, 4 * ((ks0 + 1) & 1) + g) + 128 * ((ks0 + 1) >> 1);
  int v_off[4];
  {
    const int vrow = 4 * g + (r16 >> 2);
    const int c0 = 2 * kDt * ds + ((r16 & 3) >> 1);
#pragma unroll
    for (int u = 0; u < 4; ++u) v_off[u] = vrow * kRowBytes + 16 * swz(vrow, c0 + 2 * u) + 8 * (r16 & 1);
  }
  // Complete the operand loads here: otherwise the compiler waits for them inside the
  // loop, where the counter also covers the in-flight row gather.
  __builtin_amdgcn_s_waitcnt(0);

  // Pipeline: rows of block j+1 and the idx of block j+2 are in flight while block j is
  // computed (requested during block j, after its QK); every wave waits for all of its
  // loads at the top of the block.
  // With NB = 3 the rows of blk+2 are also requested during block blk.  Loads complete
  // in issue order, and each block issues the idx of a later block before its rows, so at
  // the top of a block only the rows requested by the previous block may still be in
  // flight.
  constexpr int D = NB - 1;                     // blocks of rows requested ahead
  if (blk_begin < blk_end) {
    issue_keys(blk_begin);
    if (blk_begin + 1 < blk_end) issue_keys(blk_begin + 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    issue_rows(blk_begin, 0);
    if constexpr (D == 2) {
      if (blk_begin + 2 < blk_end) issue_keys(blk_begin + 2);
      if (blk_begin + 1 < blk_end) issue_rows(blk_begin + 1, 1);
    }
  }

  for (int blk = blk_begin; blk < blk_end; ++blk) {
    const int j = blk - blk_begin;
    const int buf = j % NB;
    if (D == 2 && blk + 1 < blk_end)                     // rows of blk and idx of blk+2 landed
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSlotsPerWave) : "memory");
    else                                                 // rows of blk and idx of blk+1 landed
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                                     // landed for all; oldest buffer free
    if (blk + D + 1 < blk_end) issue_keys(blk + D + 1);

    f32x4 sp = {0.f, 0.f, 0.f, 0.f};
    if (wave_active) {
      const uint8_t* kb = kvs[buf];
      // chunk 4ks+g of row r16 sits at 128*(ks/2) + 16*(((ks&1)*4 + g) ^ ((r16/2)&7)):
      // two per-lane bases (even/odd steps of this half) plus immediate offsets
      const uint8_t* kq0 = kb + k_off0;
      const uint8_t* kq1 = kb + k_off1;
      // operand reads run kKAhead steps ahead of the MFMAs that consume them
      constexpr int kKAhead = 3;
      bf16x8 kop[kQSteps];
#pragma unroll
      for (int ks = 0; ks < kQSteps; ++ks)
        kop[ks] = *reinterpret_cast<const bf16x8*>((ks & 1 ? kq1 : kq0) + 128 * (ks >> 1));
#pragma unroll
      for (int ks = 0; ks < kQSteps; ++ks) sp = mfma_bf16_16x16x32(kop[ks], qop[ks], sp);
      __builtin_amdgcn_sched_group_barrier(0x100, kKAhead, 0);
#pragma unroll
      for (int ks = 0; ks < kQSteps - kKAhead; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kKAhead, 0);
      if constexpr (DVS == 2) xch[j & 1][wv_id][lane] = sp;
    }
    // the next block's rows are requested after this block's QK, which thereby starts
    // right after the barrier
    if (blk + D < blk_end) issue_rows(blk + D, (j + D) % NB);
    if constexpr (DVS == 2) __syncthreads();             // partial S^T tiles exchanged
    if (wave_active) {
      const uint8_t* kb = kvs[buf];
      // with DVS = 2 both halves add the two partial tiles (fp32 addition commutes
      // exactly), so both hold the same S^T; lane holds head h, keys 4g+jj of the block
      f32x4 s = sp;
      if constexpr (DVS == 2) s = sp + xch[j & 1][partner][lane];
      const int4 kk4 = *reinterpret_cast<const int4*>(&keyring[j & (kKeyBufs - 1)][4 * g]);
      const bool v0 = (uint32_t)kk4.x < (uint32_t)a.Lk, v1 = (uint32_t)kk4.y < (uint32_t)a.Lk;
      const bool v2 = (uint32_t)kk4.z < (uint32_t)a.Lk, v3 = (uint32_t)kk4.w < (uint32_t)a.Lk;
      // scaled logits in log2 units (the block maximum is then one of them exactly, so a
      // lone dominant key gets p = 1 exactly)
      float sv[4] = {s[0] * sl2, s[1] * sl2, s[2] * sl2, s[3] * sl2};
      if (ballot(!(v0 & v1 & v2 & v3))) {        // some entry of the block invalid (rare)
        sv[0] = v0 ? sv[0] : -INFINITY;
        sv[1] = v1 ? sv[1] : -INFINITY;
        sv[2] = v2 ? sv[2] : -INFINITY;
        sv[3] = v3 ? sv[3] : -INFINITY;
      }
      const float bmax = wave_max16x4(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
      const bool need = bmax > m_use + kRescaleGap;
      if (ballot(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_use - bmax) : 1.f;
        if (need) m_use = bmax;
        l_lane *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) o[dt] *= alpha;
      }
      bf16x8 pb;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float pj = __builtin_amdgcn_exp2f(sv[jj] - m_use);
        l_lane += pj;
        const __bf16 hi = (__bf16)pj;
        pb[jj] = hi;
        pb[jj + 4] = (__bf16)(pj - (float)hi);
      }
      // O^T += V^T . P^T over the block's 16 keys (each key twice: hi and lo part of p)
      // V^T rows for dims 16dt..16dt+15: chunk c0 + 2dt of row vrow, at
      // v_off[dt % 4] + 128 * (dt / 4).  Each key enters twice (hi and lo part of p), so
      // the same transposed read fills both halves of the operand.
      // transposed reads run kVAhead tiles ahead of the MFMAs that consume them
      constexpr int kVAhead = 4;
      bf16x4 vt[kDt];
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) vt[dt] = lds_read_tr16(kb + v_off[dt & 3] + 128 * (dt >> 2));
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        const bf16x8 va = __builtin_shufflevector(vt[dt], vt[dt], 0, 1, 2, 3, 0, 1, 2, 3);
        o[dt] = mfma_bf16_16x16x32(va, pb, o[dt]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kVAhead, 0);
#pragma unroll
      for (int dt = 0; dt < kDt - kVAhead; ++dt) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kVAhead, 0);
    }
  }

  if (!wave_active) return;
  const float l_run = wave_sum16x4(l_lane);
  const size_t qh = ((size_t)b * a.Lq + i) * a.H + h;   // (query, head) row
  const int d0 = kDvPer * ds;
  if constexpr (!SPLIT) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    if (a.out_dtype == DSA_F32) {
      float* orow = reinterpret_cast<float*>(a.out) + qh * kMlaDv + d0;
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) *reinterpret_cast<f32x4*>(orow + 16 * dt + 4 * g) = o[dt] * inv;
    } else {
      uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + qh * kMlaDv + d0;
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[dt][e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 16 * dt + 4 * g) = v;
      }
    }
    if (a.lse && g == 0 && ds == 0) a.lse[qh] = l_run > 0.f ? (m_use + log2f(l_run)) / kLog2e : -INFINITY;
  } else {
    float* po = P.part_o + (qh * P.n_split + split) * kMlaDv + d0;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * g) = o[dt];
    if (g == 0 && ds == 0) {
      P.part_ml[(qh * P.n_split + split) * 2 + 0] = m_use;
      P.part_ml[(qh * P.n_split + split) * 2 + 1] = l_run;
    }
  }
}

// ---------------------------------------------------------------------------
// 32-key blocks (two 16-key sub-blocks) for workgroups of four waves, i.e. one query of
// 32 heads: the waves form two pairs (one per head tile); wave ds of a pair scores
// sub-block ds over all 576 latent dims, the pair exchanges the block maximum and then
// the two-part (hi, lo) bf16 probabilities through LDS, and each wave accumulates its
// 256 value dims over all 32 keys.  Compared with 16-key blocks split by latent dims, a
// V^T operand now carries 8 distinct keys (two transposed reads, no duplication), the
// hi and lo parts of p are two MFMAs on the same operand, and each 32 keys take three
// barriers and one max reduction instead of four and two.
// ---------------------------------------------------------------------------
// NB = latent row buffers: block j is computed from buffer j % NB while the rows of
// blocks j+1 .. j+NB-1 are in flight.  NB = 2 leaves room for two workgroups per CU (the
// prefill grids); NB = 4 takes most of the LDS for one workgroup per CU with three blocks
// (108 KB) in flight, for the few long-latency workgroups of decode.  The idx ring runs
// 2 NB - 2 blocks ahead, so a block's entries have landed before its rows are requested.
//
// KV8: the latent cache holds OCP E4M3 codes (576 per row) and one fp32 scale per row.
// The gathered code rows (18 KB per block) land in NB staging buffers with the block's 32
// scales; after the block barrier every thread converts its share of the block exactly to
// bf16 (hardware fp8 -> f32 conversion, then bf16, both exact) into one swizzled bf16
// buffer that the unchanged QK and PV code reads.  The scale of key s factors out of its
// dot products: it multiplies the key's score, and the key's probability enters the value
// product as p * scale (the denominator l sums p).
//
// NQ = queries per workgroup that share one idx row (the MTP draft queries of a sequence,
// idx_q_stride 0): 4 NQ waves, four per query.  The rows of a block are gathered once, by
// the four waves of query slot 0, and every query's waves compute from the same buffers;
// with NQ = 2 the two queries' chains share each SIMD (two waves per SIMD) instead of
// running in two workgroups that gather the same rows.
template <bool SPLIT, int NB, bool KV8, int NQ>
__global__ __launch_bounds__(256 * NQ) __attribute__((amdgpu_waves_per_eu(NB == 2 || NQ == 2 ? 2 : 1)))
void mla_attn32_kernel(MlaParams P) {
  constexpr int NW = 4 * NQ;                     // waves per workgroup
  constexpr int NWL = 4;                         // waves that gather the rows (query slot 0)
  constexpr int NT = 64 * NW;                    // threads per workgroup
  constexpr int kDt = 16;                        // 16-dim output tiles per wave (256 dims)
  constexpr int kQSteps = 18;                    // 32-dim QK steps over the 576 latent dims
  constexpr int kDma = KV8 ? kDmaPerBlk2 / 2 : kDmaPerBlk2;   // 1 KB loads per block (18 / 36)
  constexpr int kSlots = (kDma + NWL - 1) / NWL; // per loading wave (5, 5, 4, 4 / 9)
  constexpr int kKeyAhead = 2 * NB - 2;          // idx blocks requested ahead of compute
  constexpr int kKeyBufs2 = NB == 2 ? 4 : 8;     // ring slots (j .. j + kKeyAhead in use)
  static_assert((NB & (NB - 1)) == 0 && kKeyBufs2 > kKeyAhead, "ring sizes");
  constexpr int kStgBytes = kBlk2Bytes / 2;      // 32 rows of 576 codes
  constexpr int kRowLds = KV8 ? NB * kStgBytes + kBlk2Bytes : NB * kBlk2Bytes;
  __shared__ __attribute__((aligned(16))) uint8_t lrows[kRowLds];
  __shared__ __attribute__((aligned(16))) float sclring[KV8 ? kKeyBufs2 : 1][kBlk2];
  __shared__ __attribute__((aligned(16))) int keyring[kKeyBufs2][kBlk2];
  __shared__ __attribute__((aligned(16))) float xm[NW][64];     // block maxima, then l
  __shared__ __attribute__((aligned(16))) i32x4 xp[NW][64];     // packed (hi, lo) p
  const AttnArgs& a = P.a;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int wv_id = uniform(tid >> 6);
  const int qs = wv_id >> 2;                     // query slot
  const int wq = wv_id & 3;                      // wave within the query
  const int hpq = a.H / 16;                      // head tiles per query (1 or 2)
  const int ng = P.n_groups;
  int grp;
  {
    const int bid = blockIdx.x, xcd = bid & 7, jj = bid >> 3;
    const int per = ng >> 3, rem = ng & 7;
    grp = (xcd < rem) ? xcd * (per + 1) + jj : rem * (per + 1) + (xcd - rem) * per + jj;
  }
  const int split = blockIdx.y;
  const int gps = a.Lq / NQ;                     // query groups per sequence
  const int b = grp / gps;
  const int i = (grp - b * gps) * NQ + qs;       // this wave's query
  const int ht = wq % hpq;                       // head tile
  const int ds = wq / hpq;                       // sub-block scored, value half accumulated
  const bool wave_active = wq < 2 * hpq;
  const int partner = 4 * qs + (ds == 0 ? wq + hpq : wq - hpq);   // wave index
  const int32_t* idx_row = a.idx_q_stride ? a.idx + (size_t)b * a.Lq * a.idx_q_stride + (size_t)i * a.idx_q_stride
                                          : a.idx + (size_t)b * a.topk;
  const int n_blk_total = (a.topk + kBlk2 - 1) / kBlk2;
  const int blk_begin = split * P.blocks_per_split;
  const int blk_end = min(n_blk_total, blk_begin + P.blocks_per_split);
  const int nb = blk_end - blk_begin;
  constexpr int kElemBytes = KV8 ? 1 : 2;
  const uint8_t* kvbase = reinterpret_cast<const uint8_t*>(a.k) + (size_t)b * a.Lk * a.k_row_stride * kElemBytes;
  const uint32_t row_bytes32 = (uint32_t)(a.k_row_stride * kElemBytes);
  const float* sclbase = KV8 ? a.kv_scale + (size_t)b * a.Lk : nullptr;
  // DMA target of block t's rows (buffer t % NB), and the bf16 block the math reads
  auto dma_buf = [&](int buf) { return lrows + buf * (KV8 ? kStgBytes : kBlk2Bytes); };
  auto math_buf = [&](int buf) -> const uint8_t* { return KV8 ? lrows + NB * kStgBytes : lrows + buf * kBlk2Bytes; };
  const int my_loads = qs != 0 ? 0 : KV8 ? (wq + (kSlots - 1) * NWL < kDma ? kSlots : kSlots - 1) + 1 : kSlots;

  // idx entries of the t-th block of this range into ring slot t % 4 (lanes 0..31; every
  // wave issues the same load); positions past topk are -1
  auto issue_keys = [&](int t) {
    int* slot = &keyring[t & (kKeyBufs2 - 1)][0];
    const int pos = (blk_begin + t) * kBlk2 + lane;
    if (lane < kBlk2) {
      if (pos < a.topk) dma_4(idx_row + pos, lds_offset(slot));
      else slot[lane] = -1;
    }
  };
  // the block's 32 latent rows, loaded by the waves of query slot 0.  bf16: wave wq loads
  // key group wq (rows 8 wq + lane / 8) in the layout above, nine segment loads per block.
  // E4M3: the code rows land unswizzled at r * 576 (36 chunks per row) in 1 KB pieces, for
  // the conversion to bf16.
  constexpr int kRowChunks = KV8 ? kChunks / 2 : kChunks;
  int dma_row[KV8 ? kSlots : 1];
  uint32_t dma_off[KV8 ? kSlots : 1];
  if constexpr (KV8) {
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const int piece = (wq + u * NWL) * 64 + lane;
      const int r = min(piece / kRowChunks, kBlk2 - 1);   // loads past the block are skipped
      dma_row[u] = r;
      dma_off[u] = 16 * (piece - r * kRowChunks);
    }
  }
  const int dr = lane >> 3;
  const uint32_t dchunk = 16u * (uint32_t)((lane & 7) ^ sw8(dr));
  const uint8_t* row_src = kvbase;                       // this wave's row, set by the first part
  // loads u0 .. u1-1 of this wave for the t-th block (KV8: the first part also gathers the
  // block's 32 scales, every wave the same)
  auto issue_rows = [&](int t, int buf, auto u0c, auto u1c) {
    constexpr int u0 = decltype(u0c)::value, u1 = decltype(u1c)::value;
    const int* slot = &keyring[t & (kKeyBufs2 - 1)][0];
    if (qs != 0) return;                             // wave-uniform
    if constexpr (KV8) {
      if constexpr (u0 == 0) {
        if (lane < kBlk2) {
          const uint32_t kk = (uint32_t)slot[lane] < (uint32_t)a.Lk ? (uint32_t)slot[lane] : 0u;
          dma_4(sclbase + kk, lds_offset(&sclring[t & (kKeyBufs2 - 1)][0]));
        }
      }
      int key[u1 - u0];
#pragma unroll
      for (int u = u0; u < u1; ++u) key[u - u0] = slot[dma_row[u]];
#pragma unroll
      for (int u = u0; u < u1; ++u) {
        if (wq + u * NWL < kDma) {                       // wave-uniform
          const uint32_t kk = (uint32_t)key[u - u0] < (uint32_t)a.Lk ? (uint32_t)key[u - u0] : 0u;
          dma_16(kvbase + (uint64_t)kk * row_bytes32 + dma_off[u], lds_offset(dma_buf(buf) + (wq + u * NWL) * 1024));
        }
      }
    } else {
      if constexpr (u0 == 0) {
        const uint32_t key = (uint32_t)slot[8 * wq + dr];
        row_src = kvbase + (uint64_t)(key < (uint32_t)a.Lk ? key : 0u) * row_bytes32 + dchunk;   // invalid: masked later
      }
      dma_group_segs<u0, u1>(row_src, lds_offset(dma_buf(buf) + wq * kGroupBytes));
    }
  };
  using C0 = Phase<0>;
  using C3 = Phase<KV8 ? 2 : 3>;
  using C6 = Phase<KV8 ? 4 : 6>;
  using C9 = Phase<kSlots>;

  for (int t = 0; t < kKeyAhead && t < nb; ++t) issue_keys(t);
  // Q^T operand over all 576 dims: head h, dims [32 ks + 8 g, +8)
  const int h = ht * 16 + r16;
  bf16x8 qop[kQSteps];
  {
    const bf16x8* qrow = reinterpret_cast<const bf16x8*>(
        reinterpret_cast<const uint16_t*>(a.q) + (((size_t)b * a.Lq + i) * a.H + (wave_active ? h : 0)) * kMlaD);
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) qop[ks] = qrow[4 * ks + g];
  }
  f32x4 o[kDt];
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_use = -kMaxStart, l_lane = 0.f;
  const float sl2 = a.sm_scale * kLog2e;
  // K operand of row r16 of sub-block ds (group 2 ds + r16 / 8, row r16 % 8): chunk 4 ks + g
  int k_off0, k_off1;
  {
    const int w = 2 * ds + (r16 >> 3), r = r16 & 7;
    k_off0 = w * kGroupBytes + r * 128 + 16 * (g ^ sw8(r));
    k_off1 = w * kGroupBytes + r * 128 + 16 * ((4 + g) ^ sw8(r));
  }
  // V^T operand of value dims 256 ds + 16 dt ..: key row 4 g + r16 / 4 of sub-block 0
  // (sub-block 1 is two groups on), chunk 32 ds + 8 (dt / 4) + 2 (dt % 4) + (r16 % 4) / 2,
  // half r16 % 2
  int v_off[4];
  {
    const int w = g >> 1, r = 4 * (g & 1) + (r16 >> 2), bb = (r16 & 3) >> 1, hh = r16 & 1;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      v_off[m] = w * kGroupBytes + 4 * ds * kSegBytes + r * 128 + 16 * ((2 * m + bb) ^ sw8(r)) + 8 * hh;
  }
  __builtin_amdgcn_s_waitcnt(0);                 // operands and the first idx entries
  if (nb > 0) {
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NB - 1; ++t)
      if (t < nb) issue_rows(t, t, C0{}, C9{});
  }

  for (int j = 0; j < nb; ++j) {
    const int buf = j & (NB - 1);
    const int nbuf = (j + NB - 1) & (NB - 1);
    if constexpr (NB == 2) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // rows of j, idx of j+2 and before
    } else {
      // loads this wave issued after the rows of block j: those of the iterations
      // t = j-NB+2 .. j-1 (idx of block t + kKeyAhead, rows of block t + NB - 1; the
      // prologue issued rows only)
      int after = 0;
#pragma unroll
      for (int d = NB - 2; d >= 1; --d) {
        const int t = j - d;
        after += (t + NB - 1 < nb) ? my_loads : 0;
        after += (t >= 0 && t + kKeyAhead < nb) ? 1 : 0;
      }
      wait_vm_at_most<(NB - 2) * (kSlots + (KV8 ? 2 : 1))>(uniform(after));
    }
    __syncthreads();                                     // B1: landed for all; buffer of j-1 free
    // the next block's rows go out in three parts spread over the block (every wave of
    // the CU would otherwise queue all of its loads at the same moment)
    if (j + kKeyAhead < nb) issue_keys(j + kKeyAhead);
    if (j + NB - 1 < nb) issue_rows(j + NB - 1, nbuf, C0{}, C3{});
    if constexpr (KV8) {
      // the block's codes to bf16: piece p (16 codes of row p / 36) -> chunks 2c, 2c + 1
      const uint8_t* stg = dma_buf(buf);
      uint8_t* dst = lrows + NB * kStgBytes;
#pragma unroll
      for (int u = 0; u < (kStgBytes / 16 + NT - 1) / NT; ++u) {
        const int pc = tid + NT * u;
        if (pc < kStgBytes / 16) {
          const int r = pc / kRowChunks, c = pc - r * kRowChunks;
          const i32x4 w = *reinterpret_cast<const i32x4*>(stg + 16 * pc);
          i32x4 lo, hi;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            const f32x2 f0 = __builtin_amdgcn_cvt_pk_f32_fp8(w[e], false);
            const f32x2 f1 = __builtin_amdgcn_cvt_pk_f32_fp8(w[e], true);
            const int v0 = (int)pack_bf16x2(f0.x, f0.y), v1 = (int)pack_bf16x2(f1.x, f1.y);
            if (e < 2) { lo[2 * e] = v0; lo[2 * e + 1] = v1; }
            else { hi[2 * e - 4] = v0; hi[2 * e - 3] = v1; }
          }
          *reinterpret_cast<i32x4*>(dst + blk_chunk_off(r, 2 * c)) = lo;
          *reinterpret_cast<i32x4*>(dst + blk_chunk_off(r, 2 * c + 1)) = hi;
        }
      }
      __syncthreads();                                   // B1b: the bf16 block is complete
    }
    const uint8_t* kb = math_buf(buf);
    float sv[4];
    f32x4 kscale4 = {1.f, 1.f, 1.f, 1.f};           // KV8: the scales of this lane's keys
    float own_max = -INFINITY;
    // Issue priority of the waves sharing a SIMD (two workgroups per CU in prefill):
    // the score -> block maximum -> probabilities chain, whose steps end in the
    // exchange barriers, goes first (2 for the K reads, score MFMAs and maximum, 1 for
    // the probabilities); the value MFMAs (16 independent accumulators) and the row
    // loads of the next block fill the issue slots left over (0).  Timed at 128K:
    // 3% faster per layer than equal priorities, identical output.
    __builtin_amdgcn_s_setprio(2);
    if (wave_active) {
      // S^T of sub-block ds: two independent chains (even and odd steps)
      constexpr int kKAhead = 4;
      bf16x8 kop[kQSteps];
#pragma unroll
      for (int ks = 0; ks < kQSteps; ++ks)
        kop[ks] = *reinterpret_cast<const bf16x8*>(kb + (ks & 1 ? k_off1 : k_off0) + kSegBytes * (ks >> 1));
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kQSteps; ks += 2) {
        s0 = mfma_bf16_16x16x32(kop[ks], qop[ks], s0);
        s1 = mfma_bf16_16x16x32(kop[ks + 1], qop[ks + 1], s1);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kKAhead, 0);
#pragma unroll
      for (int ks = 0; ks < kQSteps - kKAhead; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kKAhead, 0);
      const f32x4 s = s0 + s1;
      // lane holds head h, keys 16 ds + 4 g + jj of the block
      const int4 kk4 = *reinterpret_cast<const int4*>(&keyring[j & (kKeyBufs2 - 1)][16 * ds + 4 * g]);
      if constexpr (KV8) {
        kscale4 = *reinterpret_cast<const f32x4*>(&sclring[j & (kKeyBufs2 - 1)][16 * ds + 4 * g]);
        sv[0] = s[0] * kscale4[0] * sl2;
        sv[1] = s[1] * kscale4[1] * sl2;
        sv[2] = s[2] * kscale4[2] * sl2;
        sv[3] = s[3] * kscale4[3] * sl2;
      } else {
        sv[0] = s[0] * sl2;
        sv[1] = s[1] * sl2;
        sv[2] = s[2] * sl2;
        sv[3] = s[3] * sl2;
      }
      const uint32_t kmax = max(max((uint32_t)kk4.x, (uint32_t)kk4.y), max((uint32_t)kk4.z, (uint32_t)kk4.w));
      if (ballot(kmax >= (uint32_t)a.Lk)) {      // some entry invalid (rare)
        sv[0] = (uint32_t)kk4.x < (uint32_t)a.Lk ? sv[0] : -INFINITY;
        sv[1] = (uint32_t)kk4.y < (uint32_t)a.Lk ? sv[1] : -INFINITY;
        sv[2] = (uint32_t)kk4.z < (uint32_t)a.Lk ? sv[2] : -INFINITY;
        sv[3] = (uint32_t)kk4.w < (uint32_t)a.Lk ? sv[3] : -INFINITY;
      }
      own_max = wave_max16x4(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
      xm[wv_id][lane] = own_max;
    }
    __builtin_amdgcn_s_setprio(1);
    if (j + NB - 1 < nb) issue_rows(j + NB - 1, nbuf, C3{}, C6{});
    __syncthreads();                                     // B2: block maxima exchanged
    if (wave_active) {
      // both waves of the pair see the same two maxima, so they raise m_use identically
      const float bmax = fmaxf(own_max, xm[partner][lane]);
      const bool need = bmax > m_use + kRescaleGap;
      if (ballot(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_use - bmax) : 1.f;
        if (need) m_use = bmax;
        l_lane *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) o[dt] *= alpha;
      }
      float pj[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        pj[jj] = __builtin_amdgcn_exp2f(sv[jj] - m_use);
        l_lane += pj[jj];
        if constexpr (KV8) pj[jj] *= kscale4[jj];      // weight of the key's code row
      }
      // p = hi + lo, hi = RNE_bf16(p), lo = RNE_bf16(p - hi)
      const uint32_t h01 = pack_bf16x2(pj[0], pj[1]), h23 = pack_bf16x2(pj[2], pj[3]);
      const uint32_t l01 = pack_bf16x2(pj[0] - __uint_as_float(h01 << 16), pj[1] - __uint_as_float(h01 & 0xffff0000u));
      const uint32_t l23 = pack_bf16x2(pj[2] - __uint_as_float(h23 << 16), pj[3] - __uint_as_float(h23 & 0xffff0000u));
      xp[wv_id][lane] = i32x4{(int)h01, (int)h23, (int)l01, (int)l23};
    }
    __builtin_amdgcn_s_setprio(0);
    if (j + NB - 1 < nb) issue_rows(j + NB - 1, nbuf, C6{}, C9{});
    __syncthreads();                                     // B3: probabilities exchanged
    if (wave_active) {
      const i32x4 mine = xp[wv_id][lane], other = xp[partner][lane];
      const i32x4 p0 = ds == 0 ? mine : other, p1 = ds == 0 ? other : mine;   // sub-blocks 0, 1
      const bf16x8 pb_hi = __builtin_bit_cast(bf16x8, i32x4{p0[0], p0[1], p1[0], p1[1]});
      const bf16x8 pb_lo = __builtin_bit_cast(bf16x8, i32x4{p0[2], p0[3], p1[2], p1[3]});
      // O^T += V^T . P^T: K slots 8g..8g+3 are keys 4g.. of sub-block 0, 8g+4.. those of 1
      constexpr int kVAhead = 4;
      bf16x4 vt0[kDt], vt1[kDt];
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        vt0[dt] = lds_read_tr16(kb + v_off[dt & 3] + kSegBytes * (dt >> 2));
        vt1[dt] = lds_read_tr16(kb + 2 * kGroupBytes + v_off[dt & 3] + kSegBytes * (dt >> 2));
      }
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        const bf16x8 va = __builtin_shufflevector(vt0[dt], vt1[dt], 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = mfma_bf16_16x16x32(va, pb_hi, o[dt]);
        o[dt] = mfma_bf16_16x16x32(va, pb_lo, o[dt]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVAhead, 0);
#pragma unroll
      for (int dt = 0; dt < kDt - kVAhead; ++dt) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * kVAhead, 0);
    }
  }

  // l over the whole block range: each wave summed its own sub-block; add in sub-block order
  const float l_own = wave_sum16x4(l_lane);
  __syncthreads();                                       // xm free
  if (wave_active) xm[wv_id][lane] = l_own;
  __syncthreads();
  if (!wave_active) return;
  const float l_other = xm[partner][lane];
  const float l_run = ds == 0 ? l_own + l_other : l_other + l_own;
  const size_t qh = ((size_t)b * a.Lq + i) * a.H + h;
  const int d0 = 256 * ds;
  if constexpr (!SPLIT) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    if (a.out_dtype == DSA_F32) {
      float* orow = reinterpret_cast<float*>(a.out) + qh * kMlaDv + d0;
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) *reinterpret_cast<f32x4*>(orow + 16 * dt + 4 * g) = o[dt] * inv;
    } else {
      uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + qh * kMlaDv + d0;
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[dt][e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 16 * dt + 4 * g) = v;
      }
    }
    if (a.lse && g == 0 && ds == 0) a.lse[qh] = l_run > 0.f ? (m_use + log2f(l_run)) / kLog2e : -INFINITY;
  } else {
    float* po = P.part_o + (qh * P.n_split + split) * kMlaDv + d0;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * g) = o[dt];
    if (g == 0 && ds == 0) {
      P.part_ml[(qh * P.n_split + split) * 2 + 0] = m_use;
      P.part_ml[(qh * P.n_split + split) * 2 + 1] = l_run;
    }
  }
}

// Combine split partials: one workgroup (128 threads x 4 dims) per (query, head).  All
// partials (at most kMaxSplit) are requested before any is used.
constexpr int kMaxSplit = 8;
__global__ __launch_bounds__(128) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml, int n_split,
                                                          void* out, int out_dtype, float* lse) {
  const size_t qh = blockIdx.x;
  const float* ml = part_ml + qh * n_split * 2;
  // slots past n_split re-read the last partial and get weight 0
  float m[kMaxSplit], l[kMaxSplit];
  f32x4 v[kMaxSplit];
#pragma unroll
  for (int sp = 0; sp < kMaxSplit; ++sp) {
    const int spc = min(sp, n_split - 1);
    m[sp] = ml[2 * spc];
    l[sp] = ml[2 * spc + 1];
    v[sp] = *reinterpret_cast<const f32x4*>(part_o + (qh * n_split + spc) * kMlaDv + 4 * threadIdx.x);
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxSplit; ++sp) M = fmaxf(M, m[sp]);
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < kMaxSplit; ++sp) {
    const float sc = (sp >= n_split || m[sp] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[sp] - M);
    L += sc * l[sp];
    acc += sc * v[sp];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (out_dtype == DSA_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + qh * kMlaDv + 4 * threadIdx.x) = acc * inv;
  } else {
    bf16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (__bf16)(acc[e] * inv);
    *reinterpret_cast<bf16x4*>(reinterpret_cast<uint16_t*>(out) + qh * kMlaDv + 4 * threadIdx.x) = r;
  }
  if (lse && threadIdx.x == 0) lse[qh] = L > 0.f ? (M + log2f(L)) / kLog2e : -INFINITY;
}

// Reference-size fp32 attention: one workgroup per (query, head); logits in LDS.
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  extern __shared__ float sm[];
  float* qv = sm;                 // [Dqk]
  float* lg = sm + a.Dqk;         // [k]
  __shared__ float red[2][4];
  const int qh = blockIdx.x;
  const int h = qh % a.H;
  const int qrow = qh / a.H;      // b * Lq + i
  const int b = qrow / a.Lq, i = qrow - b * a.Lq;
  const int kvh = h / (a.H / a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wv_id = tid >> 6;
  const int32_t* idx_row = a.idx_q_stride ? a.idx + (size_t)b * a.Lq * a.idx_q_stride + (size_t)i * a.idx_q_stride
                                          : a.idx + (size_t)b * a.topk;
  const float* q = reinterpret_cast<const float*>(a.q) + (size_t)qh * a.Dqk;
  for (int d = tid; d < a.Dqk; d += 256) qv[d] = q[d];
  __syncthreads();
  const float* kb = reinterpret_cast<const float*>(a.k) + (size_t)b * a.Lk * a.k_row_stride + (size_t)kvh * a.Dqk;
  const float* vb = reinterpret_cast<const float*>(a.v) + (size_t)b * a.Lk * a.v_row_stride + (size_t)kvh * a.Dv;
  float lmax = -INFINITY;
  for (int j = tid; j < a.topk; j += 256) {
    const int key = idx_row[j];
    float x = -INFINITY;
    if (key >= 0 && key < a.Lk) {
      const float* kr = kb + (size_t)key * a.k_row_stride;
      float d = 0.f;
      for (int e = 0; e < a.Dqk; ++e) d = fmaf(qv[e], kr[e], d);
      x = d * a.sm_scale;
    }
    lg[j] = x;
    lmax = fmaxf(lmax, x);
  }
  for (int off = 32; off > 0; off >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, off));
  if (lane == 0) red[0][wv_id] = lmax;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  float lsum = 0.f;
  for (int j = tid; j < a.topk; j += 256) {
    const float p = (lg[j] == -INFINITY) ? 0.f : expf(lg[j] - M);
    lg[j] = p;
    lsum += p;
  }
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
  if (lane == 0) red[1][wv_id] = lsum;
  __syncthreads();
  const float L = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* orow = reinterpret_cast<float*>(a.out) + (size_t)qh * a.Dv;
  for (int d = tid; d < a.Dv; d += 256) {
    float acc = 0.f;
    for (int j = 0; j < a.topk; ++j) {
      const int key = idx_row[j];
      if (key >= 0 && key < a.Lk && lg[j] != 0.f) acc = fmaf(lg[j], vb[(size_t)key * a.v_row_stride + d], acc);
    }
    orow[d] = acc * inv;
  }
  if (a.lse && tid == 0) a.lse[qh] = L > 0.f ? M + logf(L) : -INFINITY;
}

struct MlaPlan {
  int nq, dvs, nw, n_groups, n_split, bps;
  bool k32;           // mla_attn32_kernel (32-key blocks, one query or one pair sharing an idx row per workgroup)
  bool deep;          // its four-buffer form: one workgroup per CU, three blocks in flight
  size_t off_o, off_ml, total;
};

static MlaPlan plan_mla(int B, int Lq, int k, int H, int64_t idx_q_stride) {
  MlaPlan p;
  p.nq = 1;
  p.k32 = H <= 32;          // one query's heads fit two wave pairs
  if (idx_q_stride == 0 && !p.k32) {  // queries of a sequence share one row: batch them per workgroup
    p.nq = Lq;
    while (p.nq > 1 && (p.nq * (H / 16) * 2 > 8 || Lq % p.nq)) --p.nq;
  } else if (idx_q_stride == 0 && Lq % 2 == 0 && (int64_t)B * (Lq / 2) <= 256) {
    p.nq = 2;               // pairs of queries gather their shared rows once (four-buffer grid)
  }
  // each wave holds 16 heads x 256 value dims; at most 8 waves per workgroup
  p.dvs = 2;
  p.nw = p.nq * (H / 16) * p.dvs;
  p.n_groups = B * (Lq / p.nq);
  const int n_blk = (k + (p.k32 ? kBlk2 : kBlk) - 1) / (p.k32 ? kBlk2 : kBlk);
  int split = 1;
  // few query rows (decode): one deep workgroup per CU, the keys split to reach ~256 of
  // them; otherwise split to reach ~1024 two-buffer workgroups
  p.deep = p.k32 && p.n_groups <= 256;
  const int target = p.deep ? 256 : 1024;
  if (p.n_groups < target) {
    // paired queries: at most one grid of 256 workgroups, so the partials (128 KB per
    // workgroup at 32 heads) stay within 32 MiB
    split = p.nq == 2 ? target / p.n_groups : (target + p.n_groups - 1) / p.n_groups;
    if (split > kMaxSplit) split = kMaxSplit;
    if (split > n_blk) split = n_blk;
  }
  p.bps = (n_blk + split - 1) / split;
  p.n_split = (n_blk + p.bps - 1) / p.bps;
  const size_t rows = (size_t)B * Lq * H;
  p.off_o = 0;
  p.off_ml = 0;
  p.total = 0;
  if (p.n_split > 1) {
    p.off_o = 0;
    p.off_ml = (rows * p.n_split * kMlaDv * sizeof(float) + 255) / 256 * 256;
    p.total = p.off_ml + (rows * p.n_split * 2 * sizeof(float) + 255) / 256 * 256;
  }
  return p;
}

size_t sparse_attn_ws(int B, int Lq, int k, int H, int64_t idx_q_stride, int dtype) {
  if (dtype != DSA_BF16) return 0;
  return plan_mla(B, Lq, k, H, idx_q_stride).total;
}

hipError_t launch_sparse_attn(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  if (a.dtype == DSA_F32) {
    const size_t smem = (size_t)(a.Dqk + a.topk) * sizeof(float);
    attn_f32_kernel<<<a.B * a.Lq * a.H, 256, smem, s>>>(a);
    return hipGetLastError();
  }
  const MlaPlan pl = plan_mla(a.B, a.Lq, a.topk, a.H, a.idx_q_stride);
  if (ws_bytes < pl.total) return hipErrorInvalidValue;
  MlaParams P;
  P.a = a;
  P.nq = pl.nq;
  P.n_groups = pl.n_groups;
  P.n_split = pl.n_split;
  P.blocks_per_split = pl.bps;
  P.part_o = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + pl.off_o);
  P.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + pl.off_ml);
  dim3 grid(pl.n_groups, pl.n_split);
  const bool split = pl.n_split > 1;
  if (a.kv8) {   // E4M3 latent rows: the 32-key kernel only (checked by the caller)
    if (pl.deep && pl.nq == 2) {
      if (split) mla_attn32_kernel<true, 4, true, 2><<<grid, 512, 0, s>>>(P);
      else mla_attn32_kernel<false, 4, true, 2><<<grid, 512, 0, s>>>(P);
    } else if (pl.deep) {
      if (split) mla_attn32_kernel<true, 4, true, 1><<<grid, 256, 0, s>>>(P);
      else mla_attn32_kernel<false, 4, true, 1><<<grid, 256, 0, s>>>(P);
    } else {
      if (split) mla_attn32_kernel<true, 2, true, 1><<<grid, 256, 0, s>>>(P);
      else mla_attn32_kernel<false, 2, true, 1><<<grid, 256, 0, s>>>(P);
    }
  } else if (pl.k32 && pl.deep && pl.nq == 2) {
    if (split) mla_attn32_kernel<true, 4, false, 2><<<grid, 512, 0, s>>>(P);
    else mla_attn32_kernel<false, 4, false, 2><<<grid, 512, 0, s>>>(P);
  } else if (pl.k32 && pl.deep) {
    if (split) mla_attn32_kernel<true, 4, false, 1><<<grid, 256, 0, s>>>(P);
    else mla_attn32_kernel<false, 4, false, 1><<<grid, 256, 0, s>>>(P);
  } else if (pl.k32) {
    if (split) mla_attn32_kernel<true, 2, false, 1><<<grid, 256, 0, s>>>(P);
    else mla_attn32_kernel<false, 2, false, 1><<<grid, 256, 0, s>>>(P);
  } else if (pl.nw <= 4) {
    if (split) mla_attn_kernel<4, 2, 3, true, 2><<<grid, 256, 0, s>>>(P);
    else mla_attn_kernel<4, 2, 3, false, 2><<<grid, 256, 0, s>>>(P);
  } else {
    if (split) mla_attn_kernel<8, 2, 2, true, 3><<<grid, 512, 0, s>>>(P);
    else mla_attn_kernel<8, 2, 2, false, 2><<<grid, 512, 0, s>>>(P);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.n_split == 1) return e;
  mla_combine_kernel<<<a.B * a.Lq * a.H, 128, 0, s>>>(P.part_o, P.part_ml, pl.n_split, a.out, a.out_dtype, a.lse);
  return hipGetLastError();
}

}  // namespace dsa
