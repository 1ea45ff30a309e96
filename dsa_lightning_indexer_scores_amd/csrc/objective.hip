// The group-centroid objective of the kept indexer, backward (training; gfx950).
//
// GLM-5.2 技术报告速览, section "IndexShare": reusing one index set across a group of layers
// loses accuracy when each indexer was trained for its own layer only, so the kept indexer
// is fit, by KL, to the centroid pbar_t = (1 / (m + 1)) sum_j p_t^(l+j) of the head-averaged
// attention distributions of the m + 1 layers it serves.  Read here in the sparse form:
// both distributions live on the query's index row S_t, and the loss of row t is
// KL(pbar_t || pi_t) with pi_t = softmax over S_t of the indexer scores
//   I[t, s] = sum_j w[t, j] ReLU(q[t, j] . k[s]).
// Its gradient with respect to I[t, s] is pi - pbar; with x = q[t, j] . k[s] and
// c[j, s] = (pi - pbar)[s] w[t, j] [x > 0]:
//   dw[t, j] = sum_s (pi - pbar)[s] ReLU(x),   dq[t, j] = sum_s c[j, s] k[s],
//   dk[s]   += sum_t sum_j c[j, s] q[t, j]   (accumulated over the rows that selected s).
//
// attn_probs32_kernel: one layer's head-averaged distribution on S_t, recomputed from the
// layer's queries, latent rows and log-sum-exp (that of dsa_sparse_attn), accumulated
// with a weight, in the gathered 32-key blocks of the sparse attention (mla_blocks.hpp).
//
// indexer_kl_kernel: one workgroup per query row (75 KB of LDS: two per CU), selected keys
// in tiles of 64 gathered to LDS (row-major for the scores, transposed for dq).  Pass 1 scores every tile (wave w
// owns heads 16w..16w+15; MFMA 16x16x32 bf16, fp32 accumulation) and keeps I in LDS; the
// softmax, the loss and g = pi - pbar follow.  Pass 2 rescores each tile, forms c (rounded
// to bf16 for the matrix cores), accumulates dw in fp32 and runs two more contractions:
// dq (heads x dims over the tile's keys) in registers, and dk (keys x dims over the heads),
// added in 64-bit fixed point to a workspace (dk_fix_add_kernel adds it to dk), so that dk
// does not depend on the order in which rows arrive.
#include "dsa_common.hpp"
#include "dsa_launch.hpp"
#include "mla_blocks.hpp"
#include "../../include/dsa.h"

namespace dsa {

namespace {
constexpr int kDI = 128;          // indexer head dim
constexpr int kTile = 64;         // selected keys per tile
// LDS tiles are unpadded; their 16-byte chunks are XOR-swizzled by the row so that the 16
// rows one operand read touches start in different banks.  sw128: [rows][128] bf16 (the
// row-major key tile), sw64: [rows][64] bf16 (transposed and coefficient tiles).
__device__ __forceinline__ int sw128(int row, int col) {
  return row * 128 + ((((col >> 3) ^ (row & 15)) << 3) | (col & 7));
}
__device__ __forceinline__ int sw64(int row, int col) {
  return row * 64 + ((((col >> 3) ^ (row & 7)) << 3) | (col & 7));
}
}  // namespace

// ---------------------------------------------------------------------------
// One layer's head-averaged attention distribution on each query's index row, for the
// group centroid of the kept indexer's training (dsa_attn_probs):
//   P[r, i] += alpha / H sum_h exp(sm_scale q[r, h] . K[S_r[i]] - lse[r, h]).
// The gather and the score MFMAs are those of the sparse attention's mla_attn32_kernel
// (attn.hip; the block layout is in mla_blocks.hpp): two row buffers of 32 latent rows,
// the idx ring two blocks ahead, wave (ht, ds) scoring sub-block ds against head tile ht
// with Q^T in registers (here Q^T is the A operand, so a lane holds four heads of one
// key).  The log-sum-exp is known, so there is no running maximum and no exchange
// inside a block: a lane adds its four heads and two lane swaps add the four lane groups,
// and with 32 heads the second head tile's sums reach the first through LDS.
// A block's P entries are written one block later (after the next block barrier), from
// values of P loaded when the block started, so every block takes one barrier and the
// read-modify-write of P waits on no load.  Each P entry is written once per call, by
// one lane, so results do not depend on timing.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void attn_probs32_kernel(AttnProbsArgs a) {
  constexpr int NB = 2;
  constexpr int kQSteps = 18;
  constexpr int kKeyAhead = 2 * NB - 2;
  constexpr int kKeyBufs2 = 4;
  __shared__ __attribute__((aligned(16))) uint8_t lrows[NB * kBlk2Bytes];
  __shared__ __attribute__((aligned(16))) int keyring[kKeyBufs2][kBlk2];
  __shared__ float xsum[2][2][16];                 // [block parity][sub-block][key]: head tile 1
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int wv_id = uniform(tid >> 6);
  const int hpq = a.H / 16;                        // head tiles (1 or 2)
  const int ht = wv_id % hpq;
  const int ds = wv_id / hpq;
  const bool wave_active = wv_id < 2 * hpq;
  int r;                                           // query row b * Lq + i
  {
    // contiguous query ranges per XCD: neighbouring queries, whose index rows overlap,
    // share an L2 (16K, 4 layers: 10.26 -> 10.15 ms)
    const int nr = a.B * a.Lq;
    const int bid = blockIdx.x, xcd = bid & 7, jj = bid >> 3;
    const int per = nr >> 3, rem = nr & 7;
    r = (xcd < rem) ? xcd * (per + 1) + jj : rem * (per + 1) + (xcd - rem) * per + jj;
  }
  const int b = r / a.Lq;
  // the idx row of (b, i) as in dsa_sparse_attn: one per query, or one per sequence
  const int32_t* idx_row = a.idx_q_stride ? a.idx + (size_t)r * a.idx_q_stride : a.idx + (size_t)b * a.k;
  const int nb = (a.k + kBlk2 - 1) / kBlk2;
  const uint8_t* kvbase = static_cast<const uint8_t*>(a.kv) + (size_t)b * a.Lk * a.k_row_stride * 2;
  const uint32_t row_bytes32 = (uint32_t)(a.k_row_stride * 2);
  float* prow = a.P + (size_t)r * a.k;
  const float wscale = a.alpha / (float)a.H;

  // idx entries of block t into ring slot t % 4 (lanes 0..31; every wave issues the same
  // load, so its own vmcnt covers them); entries past k are -1
  auto issue_keys = [&](int t) {
    int* slot = &keyring[t & (kKeyBufs2 - 1)][0];
    const int pos = t * kBlk2 + lane;
    if (lane < kBlk2) {
      if (pos < a.k) dma_4(idx_row + pos, lds_offset(slot));
      else slot[lane] = -1;
    }
  };
  // the 32 rows of block t: wave w loads key group w (rows 8 w + lane / 8), nine segments
  const int dr = lane >> 3;
  const uint32_t dchunk = 16u * (uint32_t)((lane & 7) ^ sw8(dr));
  auto issue_rows = [&](int t, int buf) {
    const uint32_t key = (uint32_t)keyring[t & (kKeyBufs2 - 1)][8 * wv_id + dr];
    const uint8_t* src = kvbase + (uint64_t)(key < (uint32_t)a.Lk ? key : 0u) * row_bytes32 + dchunk;
    dma_group_segs<0, 9>(src, lds_offset(lrows + buf * kBlk2Bytes + wv_id * kGroupBytes));
  };

  for (int t = 0; t < kKeyAhead && t < nb; ++t) issue_keys(t);
  const int h = ht * 16 + r16;
  bf16x8 qop[kQSteps];
  {
    const bf16x8* qrow = reinterpret_cast<const bf16x8*>(
        reinterpret_cast<const uint16_t*>(a.q) + ((size_t)r * a.H + (wave_active ? h : 0)) * kMlaD);
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) qop[ks] = qrow[4 * ks + g];
  }
  const float sl2 = a.sm_scale * kLog2e;
  float lse2[4];                                   // heads 16 ht + 4 g + i
#pragma unroll
  for (int i = 0; i < 4; ++i) lse2[i] = a.lse[(size_t)r * a.H + (wave_active ? ht * 16 + 4 * g + i : 0)] * kLog2e;
  int k_off0, k_off1;
  {
    const int w = 2 * ds + (r16 >> 3), rr = r16 & 7;
    k_off0 = w * kGroupBytes + rr * 128 + 16 * (g ^ sw8(rr));
    k_off1 = w * kGroupBytes + rr * 128 + 16 * ((4 + g) ^ sw8(rr));
  }
  // lanes 0..15 of head tile 0 own slot 16 ds + r16 of every block: its P entry is the
  // loaded old value plus the wave's head sum and, with 32 heads, head tile 1's from LDS
  const bool owner = wave_active && ht == 0 && g == 0;
  const int sl = 16 * ds + r16;
  auto put = [&](int t, float own, float old) {
    float v = own;
    if (hpq == 2) v += xsum[t & 1][ds][r16];
    const int key = keyring[t & (kKeyBufs2 - 1)][sl];
    const int pos = t * kBlk2 + sl;
    if (pos < a.k && (uint32_t)key < (uint32_t)a.Lk) prow[pos] = old + wscale * v;
  };
  __builtin_amdgcn_s_waitcnt(0);                   // operands and the first idx entries
  if (nb > 0) {
    __syncthreads();
    issue_rows(0, 0);
  }
  float held = 0.f, pold = 0.f;                     // owners: the previous block's sum and old P
  for (int j = 0; j < nb; ++j) {
    const int buf = j & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // rows of j, idx of j+1, P of j-1
    __syncthreads();                                     // landed for all; buffer of j-1 free
    if (owner && j > 0) put(j - 1, held, pold);
    if (owner) pold = j * kBlk2 + sl < a.k ? prow[j * kBlk2 + sl] : 0.f;
    if (j + kKeyAhead < nb) issue_keys(j + kKeyAhead);
    if (j + 1 < nb) issue_rows(j + 1, buf ^ 1);
    if (wave_active) {
      const uint8_t* kb = lrows + buf * kBlk2Bytes;
      bf16x8 kop[kQSteps];
#pragma unroll
      for (int ks = 0; ks < kQSteps; ++ks)
        kop[ks] = *reinterpret_cast<const bf16x8*>(kb + (ks & 1 ? k_off1 : k_off0) + kSegBytes * (ks >> 1));
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kQSteps; ks += 2) {
        s0 = mfma_bf16_16x16x32(qop[ks], kop[ks], s0);
        s1 = mfma_bf16_16x16x32(qop[ks + 1], kop[ks + 1], s1);
      }
      const f32x4 s = s0 + s1;
      // lane: key 16 ds + r16, heads 16 ht + 4 g + i
      float e = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) e += __builtin_amdgcn_exp2f(s[i] * sl2 - lse2[i]);
      const float mine = wave_sum16x4(e);              // the 16 heads of the tile
      if (g == 0) {
        if (ht == 1) xsum[j & 1][ds][r16] = mine;
        else held = mine;
      }
    }
  }
  __syncthreads();                                       // head tile 1's sums of the last block
  if (owner && nb > 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // P of the last block
    put(nb - 1, held, pold);
  }
}

hipError_t launch_attn_probs(const AttnProbsArgs& a, hipStream_t s) {
  attn_probs32_kernel<<<a.B * a.Lq, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
template <int HB>
__global__ __launch_bounds__(256) void indexer_kl_kernel(IndexerKlArgs a) {
  constexpr int H = 16 * HB;
  __shared__ __attribute__((aligned(16))) __bf16 kt[kTile * kDI];     // [key][dim], sw128
  __shared__ __attribute__((aligned(16))) __bf16 ktT[kDI * kTile];    // [dim][key], sw64
  __shared__ __attribute__((aligned(16))) __bf16 qT[kDI * 64];        // [dim][head], sw64
  __shared__ __attribute__((aligned(16))) __bf16 cm[64 * kTile];      // c [head][key], sw64
  __shared__ __attribute__((aligned(16))) __bf16 cmT[kTile * 64];     // c [key][head], sw64
  __shared__ float sc[kMaxKlK];                                              // I, then pi - pbar
  __shared__ float part[4][kTile];
  __shared__ float red[8];
  __shared__ int sel[kTile];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int r = blockIdx.x;
  const int b = r / a.Lq;
  const bool active = wv < HB;                    // waves past the heads only help with loads
  const __bf16* qrow = static_cast<const __bf16*>(a.q) + (size_t)r * H * kDI;
  const __bf16* kbase = static_cast<const __bf16*>(a.kI) + (size_t)b * a.Lk * kDI;
  const float* wrow = a.w + (size_t)r * H;
  const int32_t* irow = a.idx + (size_t)r * a.k;
  const float* pbar = a.pbar + (size_t)r * a.k;

  // q^T in LDS (B operand of dk) and this wave's heads as A operands of the scores
  for (int e = tid; e < 64 * kDI; e += 256) {   // head slots past H hold zeros
    const int h = e / kDI, d = e - h * kDI;
    __bf16 v = (__bf16)0.f;
    if (h < H) v = qrow[e];
    qT[sw64(d, h)] = v;
  }
  bf16x8 aq[4];
  float wh[4];
  const int hw = active ? wv : 0;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    aq[ks] = *reinterpret_cast<const bf16x8*>(qrow + (16 * hw + l16) * kDI + 32 * ks + 8 * g4);
#pragma unroll
  for (int i = 0; i < 4; ++i) wh[i] = wrow[16 * hw + 4 * g4 + i];

  // gather tile t: the selected rows, row-major into kt and transposed into ktT (-1 and
  // out-of-range entries read row 0 and are masked by sel = -1)
  auto gather = [&](int t) {
    __syncthreads();   // the previous tile's LDS reads are done
    if (tid < kTile) {
      const int slot = t * kTile + tid;
      const int s = slot < a.k ? irow[slot] : -1;
      sel[tid] = (s >= 0 && s < a.Lk) ? s : -1;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u, key = c >> 4, ch = c & 15;
      const int s = sel[key];
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(kbase + (size_t)(s >= 0 ? s : 0) * kDI + 8 * ch);
      *reinterpret_cast<bf16x8*>(&kt[sw128(key, 8 * ch)]) = v;
#pragma unroll
      for (int e = 0; e < 8; ++e) ktT[sw64(8 * ch + e, key)] = v[e];
    }
    __syncthreads();
  };
  // x[kb] lane l: key 16 kb + l % 16 of the tile, heads 16 hw + 4 (l / 16) + i
  auto scores = [&](f32x4 (&x)[4]) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&kt[sw128(16 * kb + l16, 32 * ks + 8 * g4)]);
        acc = mfma_bf16_16x16x32(aq[ks], bv, acc);
      }
      x[kb] = acc;
    }
  };

  const int n_tiles = (a.k + kTile - 1) / kTile;
  // pass 1: I on every selected key
  for (int t = 0; t < n_tiles; ++t) {
    gather(t);
    if (active) {
      f32x4 x[4];
      scores(x);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wh[i], fmaxf(x[kb][i], 0.f), v);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (g4 == 0) part[wv][16 * kb + l16] = v;
      }
    }
    __syncthreads();
    if (tid < kTile) {
      const int slot = t * kTile + tid;
      if (slot < a.k) {
        float v = 0.f;
        for (int w = 0; w < HB; ++w) v += part[w][tid];
        sc[slot] = sel[tid] >= 0 ? v : -INFINITY;
      }
    }
  }
  __syncthreads();

  // softmax over the selected keys, the loss, and g = pi - pbar
  auto block_sum = [&](float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    __syncthreads();
    if (lane == 0) red[wv] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
  };
  float m = -INFINITY;
  for (int i = tid; i < a.k; i += 256) m = fmaxf(m, sc[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) red[4 + wv] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
  float z = 0.f;
  if (m > -INFINITY)
    for (int i = tid; i < a.k; i += 256) z += expf(sc[i] - m);
  z = block_sum(z);
  const float log_z = logf(z);
  float kl = 0.f;
  for (int i = tid; i < a.k; i += 256) {
    const float I = sc[i];
    const float p = pbar[i];
    float gi = 0.f;
    if (I > -INFINITY) {
      const float log_pi = I - m - log_z;
      gi = expf(log_pi) - p;
      if (p > 0.f) kl += p * (logf(p) - log_pi);
    }
    sc[i] = gi;
  }
  kl = block_sum(kl);
  if (tid == 0) a.loss[r] = kl;

  // pass 2: gradients
  f32x4 dq[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) dq[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dwp[4] = {0.f, 0.f, 0.f, 0.f};
  unsigned long long* dkf = a.dk_fix + (size_t)b * a.Lk * kDI;
  for (int t = 0; t < n_tiles; ++t) {
    gather(t);
    if (active) {
      f32x4 x[4];
      scores(x);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int key = 16 * kb + l16, slot = t * kTile + key;
        const float gk = (slot < a.k && sel[key] >= 0) ? sc[slot] : 0.f;
        __bf16 cv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dwp[i] = fmaf(gk, fmaxf(x[kb][i], 0.f), dwp[i]);
          const float c = x[kb][i] > 0.f ? gk * wh[i] : 0.f;
          cv[i] = (__bf16)c;
          cm[sw64(16 * wv + 4 * g4 + i, key)] = cv[i];
        }
        *reinterpret_cast<bf16x4*>(&cmT[sw64(key, 16 * wv + 4 * g4)]) = bf16x4{cv[0], cv[1], cv[2], cv[3]};
      }
    } else {
      // waves past the heads: zero coefficients so that the dk contraction over 64 head
      // slots reads zeros there
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int key = 16 * kb + l16;
        *reinterpret_cast<bf16x4*>(&cmT[sw64(key, 16 * wv + 4 * g4)]) = bf16x4{0, 0, 0, 0};
      }
    }
    __syncthreads();
    // dq (wave w: heads 16w.., all 128 dims) over the tile's 64 keys
    if (active) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&cm[sw64(16 * wv + l16, 32 * ks + 8 * g4)]);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&ktT[sw64(16 * db + l16, 32 * ks + 8 * g4)]);
          dq[db] = mfma_bf16_16x16x32(av, bv, dq[db]);
        }
      }
    }
    // dk (wave w: keys 16w.. of the tile, all 128 dims) over the 64 head slots
    {
      f32x4 acc[8];
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        if (32 * hs >= H) break;
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&cmT[sw64(16 * wv + l16, 32 * hs + 8 * g4)]);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&qT[sw64(16 * db + l16, 32 * hs + 8 * g4)]);
          acc[db] = mfma_bf16_16x16x32(av, bv, acc[db]);
        }
      }
      // acc[db] lane l: dim 16 db + l % 16, keys 16 wv + 4 (l / 16) + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * wv + 4 * g4 + i;
        const int s = sel[key];
        if (s >= 0 && t * kTile + key < a.k) {
#pragma unroll
          for (int db = 0; db < 8; ++db)
            atomicAdd(&dkf[(size_t)s * kDI + 16 * db + l16],
                      (unsigned long long)__float2ll_rn(acc[db][i] * (float)(1 << kDkFixBits)));
        }
      }
    }
  }

  if (active) {
    // dq[db] lane l: dim 16 db + l % 16, heads 16 wv + 4 (l / 16) + i
    float* dqr = a.dq + (size_t)r * H * kDI;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) dqr[(16 * wv + 4 * g4 + i) * kDI + 16 * db + l16] = dq[db][i];
    // dw: the lane's 4 heads summed over its key columns, then over the 16 lanes of the row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = dwp[i];
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (l16 == 0) a.dw[(size_t)r * H + 16 * wv + 4 * g4 + i] = v;
    }
  }
}


// dk[e] += the fixed-point sum of element e (two's complement in 64 bits)
__global__ __launch_bounds__(256) void dk_fix_add_kernel(const unsigned long long* __restrict__ fix,
                                                         float* __restrict__ dk, size_t n) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n) dk[e] += (float)((double)(long long)fix[e] * (1.0 / (double)(1ll << kDkFixBits)));
}

hipError_t launch_indexer_kl(const IndexerKlArgs& a, hipStream_t s) {
  const int rows = a.B * a.Lq;
  const size_t n_dk = (size_t)a.B * a.Lk * 128;
  hipError_t e = launch_zero(a.dk_fix, n_dk * sizeof(unsigned long long), s);
  if (e != hipSuccess) return e;
  switch (a.H_I / 16) {
    case 1: indexer_kl_kernel<1><<<rows, 256, 0, s>>>(a); break;
    case 2: indexer_kl_kernel<2><<<rows, 256, 0, s>>>(a); break;
    case 3: indexer_kl_kernel<3><<<rows, 256, 0, s>>>(a); break;
    default: indexer_kl_kernel<4><<<rows, 256, 0, s>>>(a); break;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dk_fix_add_kernel<<<(unsigned)((n_dk + 255) / 256), 256, 0, s>>>(a.dk_fix, a.dk, n_dk);
  return hipGetLastError();
}

}  // namespace dsa
