// Sparse core attention over selected positions (gfx950).
//
// GLM 5.2: Built for Long Horizon Tasks, discussion section "DSA 与 IndexShare 的组合数据流":
// each layer reads the K/V of the selected positions from its own cache and recomputes
// score, softmax and value aggregation on them only.  MLA latent form (GLM-5 technical
// report section 2.1; same discussion section): one 576-d latent row per key (512-d
// compressed KV + 64-d RoPE key); K is the whole row, V its first 512 dims, and the
// query heads are already absorbed to 576-d.
//
// MLA kernel: one workgroup per (query row group, key split); a row group is the nq
// queries that share one idx row (nq = 1, or the MTP draft queries).  Each wave owns
// 16 heads of one query.  Per 32-key block the workgroup gathers the 32 selected latent
// rows (1152 B each) into LDS once; every wave then computes
//   S^T[key, head] = K . Q^T  (bf16 MFMA 16x16x32, K from LDS, Q^T in registers),
// an online softmax per head (each lane owns one head), and
//   O^T[dv, head] += V^T . P^T  (V^T read from the row-major LDS tile with the gfx950
// transposing LDS load; P^T straight from the S^T accumulators).
#include "dsa_common.hpp"
#include "dsa_launch.hpp"
#include "../../include/dsa.h"

namespace dsa {

constexpr int kMlaD = 576;
constexpr int kMlaDv = 512;
constexpr int kBlk = 32;                       // keys per block
constexpr int kLdsRow = kMlaD * 2 + 16;        // padded LDS row (bytes)
constexpr int kPieces = kMlaD * 2 / 16;        // 72 x 16 B per row
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x4 lds_read_tr16(const uint8_t* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

struct MlaParams {
  AttnArgs a;
  int nq;            // queries sharing one idx row
  int n_groups;      // B * Lq / nq
  int n_split;
  int blocks_per_split;
  float* part_o;     // [n_groups*nq*H][n_split][512]   (n_split > 1)
  float* part_ml;    // [n_groups*nq*H][n_split][2]
};

template <int NW>
__global__ __launch_bounds__(NW * 64) void mla_attn_kernel(MlaParams P) {
  __shared__ __attribute__((aligned(16))) uint8_t kv[kBlk * kLdsRow];
  const AttnArgs& a = P.a;
  const int NT = NW * 64;
  const int tid = threadIdx.x, lane = tid & 63, wv_id = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int hpq = a.H / 16;                 // head tiles per query
  const int grp = blockIdx.x;
  const int split = blockIdx.y;
  const int qpl = a.Lq / P.nq;              // row groups per sequence
  const int b = grp / qpl;
  const int qi = wv_id / hpq;               // query of this wave within the group
  const int ht = wv_id - qi * hpq;
  const int i = (grp - b * qpl) * P.nq + qi;  // query index within the sequence
  const bool wave_active = wv_id < P.nq * hpq;
  const int32_t* idx_row = a.idx_q_stride
                               ? a.idx + (size_t)b * a.Lq * a.idx_q_stride + (size_t)((grp - b * qpl) * P.nq) * a.idx_q_stride
                               : a.idx + (size_t)b * a.topk;
  // (with a per-query idx row, nq == 1 so the group's first query is the query itself)
  const int blk_begin = split * P.blocks_per_split;
  const int n_blk_total = (a.topk + kBlk - 1) / kBlk;
  const int blk_end = min(n_blk_total, blk_begin + P.blocks_per_split);

  const uint16_t* kvbase = reinterpret_cast<const uint16_t*>(a.k) + (size_t)b * a.Lk * a.k_row_stride;

  // Q^T operand: head h, dims [32 ks + 8 g, +8)
  const int h = ht * 16 + r16;
  bf16x8 qop[18];
  {
    const int qq = wave_active ? i : 0;
    const bf16x8* qrow = reinterpret_cast<const bf16x8*>(
        reinterpret_cast<const uint16_t*>(a.q) + (((size_t)b * a.Lq + qq) * a.H + (wave_active ? h : 0)) * kMlaD);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qop[ks] = qrow[4 * ks + g];
  }
  f32x4 o[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.sm_scale * kLog2e;

  for (int blk = blk_begin; blk < blk_end; ++blk) {
    const int kb0 = blk * kBlk;
    // gather the block's latent rows (invalid entries read row 0 and are masked below)
#pragma unroll 2
    for (int p0 = 0; p0 < kBlk * kPieces; p0 += NT * 6) {
      i32x4 tmp[6];
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        const int p = p0 + u * NT + tid;
        tmp[u] = i32x4{0, 0, 0, 0};
        if (p < kBlk * kPieces) {
          const int rr = p / kPieces, c = p - rr * kPieces;
          const int pos = kb0 + rr;
          int key = pos < a.topk ? idx_row[pos] : -1;
          if (key < 0 || key >= a.Lk) key = 0;
          tmp[u] = *reinterpret_cast<const i32x4*>(kvbase + (size_t)key * a.k_row_stride + 8 * c);
        }
      }
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        const int p = p0 + u * NT + tid;
        if (p < kBlk * kPieces) {
          const int rr = p / kPieces, c = p - rr * kPieces;
          *reinterpret_cast<i32x4*>(&kv[rr * kLdsRow + 16 * c]) = tmp[u];
        }
      }
    }
    __syncthreads();

    if (wave_active) {
      // S^T for keys [0,16) and [16,32) of the block
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(&kv[r16 * kLdsRow + (32 * ks + 8 * g) * 2]);
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(&kv[(16 + r16) * kLdsRow + (32 * ks + 8 * g) * 2]);
        s0 = mfma_bf16_16x16x32(k0, qop[ks], s0);
        s1 = mfma_bf16_16x16x32(k1, qop[ks], s1);
      }
      // lane holds head h, keys 4g+i (s0) and 16+4g+i (s1)
      float sv[8];
      float bmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kk = (j < 4) ? (4 * g + j) : (16 + 4 * g + j - 4);
        const int pos = kb0 + kk;
        const int key = pos < a.topk ? idx_row[pos] : -1;
        const bool valid = key >= 0 && key < a.Lk;
        const float raw = (j < 4) ? s0[j] : s1[j - 4];
        sv[j] = valid ? raw * sl2 : -INFINITY;
        bmax = fmaxf(bmax, sv[j]);
      }
      bmax = wave_max16x4(bmax);
      const float m_new = fmaxf(m_run, bmax);
      const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
      // P is applied as bf16 hi + lo parts (p = hi + lo + O(2^-16 p)): a single bf16
      // rounding of p would cost up to 2^-8 relative on the dominant keys.
      float psum = 0.f;
      bf16x8 pb, pl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pj = (sv[j] == -INFINITY) ? 0.f : exp2f(sv[j] - m_new);
        psum += pj;
        const __bf16 hi = (__bf16)pj;
        pb[j] = hi;
        pl[j] = (__bf16)(pj - (float)hi);
      }
      psum = wave_sum16x4(psum);
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) o[dt] *= alpha;
      // O^T += V^T . P^T ; V^T operand via transposing LDS reads
      const int vrow0 = 4 * g + (r16 >> 2);
      const int vcol = 4 * (r16 & 3);
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        const bf16x4 lo = lds_read_tr16(&kv[vrow0 * kLdsRow + (16 * dt + vcol) * 2]);
        const bf16x4 hi = lds_read_tr16(&kv[(16 + vrow0) * kLdsRow + (16 * dt + vcol) * 2]);
        const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[dt] = mfma_bf16_16x16x32(va, pb, o[dt]);
        o[dt] = mfma_bf16_16x16x32(va, pl, o[dt]);
      }
    }
    __syncthreads();
  }

  if (!wave_active) return;
  const size_t qh = ((size_t)b * a.Lq + i) * a.H + h;   // (query, head) row
  if (P.n_split == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    if (a.out_dtype == DSA_F32) {
      float* orow = reinterpret_cast<float*>(a.out) + qh * kMlaDv;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) *reinterpret_cast<f32x4*>(orow + 16 * dt + 4 * g) = o[dt] * inv;
    } else {
      uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + qh * kMlaDv;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[dt][e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 16 * dt + 4 * g) = v;
      }
    }
    if (a.lse && g == 0) a.lse[qh] = l_run > 0.f ? (m_run + log2f(l_run)) / kLog2e : -INFINITY;
  } else {
    float* po = P.part_o + (qh * P.n_split + split) * kMlaDv;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * g) = o[dt];
    if (g == 0) {
      P.part_ml[(qh * P.n_split + split) * 2 + 0] = m_run;
      P.part_ml[(qh * P.n_split + split) * 2 + 1] = l_run;
    }
  }
}

// Combine split partials: one workgroup (128 threads x 4 dims) per (query, head).
__global__ __launch_bounds__(128) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml, int n_split,
                                                          void* out, int out_dtype, float* lse) {
  const size_t qh = blockIdx.x;
  const float* ml = part_ml + qh * n_split * 2;
  float M = -INFINITY;
  for (int sp = 0; sp < n_split; ++sp) M = fmaxf(M, ml[2 * sp]);
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < n_split; ++sp) {
    const float m = ml[2 * sp], l = ml[2 * sp + 1];
    const float sc = (m == -INFINITY) ? 0.f : exp2f(m - M);
    L += sc * l;
    const f32x4 v = *reinterpret_cast<const f32x4*>(part_o + (qh * n_split + sp) * kMlaDv + 4 * threadIdx.x);
    acc += sc * v;
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
  int nq, n_groups, n_split, bps;
  size_t off_o, off_ml, total;
};

static MlaPlan plan_mla(int B, int Lq, int k, int H, int64_t idx_q_stride) {
  MlaPlan p;
  p.nq = 1;
  if (idx_q_stride == 0) {  // queries of a sequence share one row: batch them per workgroup
    p.nq = Lq;
    while (p.nq > 1 && (p.nq * (H / 16) > 8 || Lq % p.nq)) --p.nq;
  }
  p.n_groups = B * (Lq / p.nq);
  const int n_blk = (k + kBlk - 1) / kBlk;
  int split = 1;
  if (p.n_groups < 1024) {       // split the keys to fill the GPU (decode)
    split = (1024 + p.n_groups - 1) / p.n_groups;
    if (split > 8) split = 8;
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
  const int nw = pl.nq * (a.H / 16);
  dim3 grid(pl.n_groups, pl.n_split);
  if (nw <= 2) mla_attn_kernel<2><<<grid, 128, 0, s>>>(P);
  else if (nw <= 4) mla_attn_kernel<4><<<grid, 256, 0, s>>>(P);
  else mla_attn_kernel<8><<<grid, 512, 0, s>>>(P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.n_split == 1) return e;
  mla_combine_kernel<<<a.B * a.Lq * a.H, 128, 0, s>>>(P.part_o, P.part_ml, pl.n_split, a.out, a.out_dtype, a.lse);
  return hipGetLastError();
}

}  // namespace dsa
