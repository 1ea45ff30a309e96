"""fp64 definitions of the indexer score, the top-k selection, sparse attention and the
IndexShare layer group (test infrastructure only; see the package docstring).

Conventions shared by every function:

* Batched rows: query i of a call with Lq queries and Lk keys sits at position
  p_i = Lk - Lq + i and may see keys s <= p_i (causality, GLM-5.2 技术报告速览,
  section "IndexShare": only key positions s <= t are legal).
* Inputs are already-decoded float64 arrays.  fp8 inputs are passed as the decoded
  code values plus their per-token fp32 scales; the dequantised value is code * scale.
"""

import numpy as np


def causal_position(Lq, Lk, i):
    """Position of query i when Lq queries are the last Lq of Lk keys."""
    return Lk - Lq + i


# ---------------------------------------------------------------------------
# Indexer score.  GLM-5.2 技术报告速览, section "IndexShare", indexer-score equation:
#   I[t, s] = sum_{j=1..H_I} w[t, j] * ReLU(q[t, j, :] . k[s, :]),   s <= t.
# ---------------------------------------------------------------------------

def _dequant(x, scale, axes):
    if scale is None:
        return np.asarray(x, dtype=np.float64)
    s = np.asarray(scale, dtype=np.float64)
    return np.asarray(x, dtype=np.float64) * s.reshape(s.shape + (1,) * axes)


def indexer_scores_rows(q, k, w, rows, Lk, q_scale=None, k_scale=None, Lq=None):
    """Scores of the selected query rows of one sequence.

    q: [Lq, H, d] float64 (codes if q_scale is given), k: [Lk, d], w: [Lq, H],
    q_scale: [Lq] or None, k_scale: [Lk] or None, rows: iterable of query indices.
    Returns [len(rows), Lk] float64 with -inf at the non-causal positions s > p_i.
    """
    Lq = q.shape[0] if Lq is None else Lq
    kk = _dequant(k, k_scale, 1)                      # [Lk, d]
    out = np.full((len(rows), Lk), -np.inf)
    for r, i in enumerate(rows):
        p = causal_position(Lq, Lk, i)
        qi = _dequant(q[i], None if q_scale is None else q_scale[i], 0)
        qi = np.asarray(qi, dtype=np.float64)         # [H, d]
        dots = qi @ kk[: p + 1].T                     # [H, p+1]   q_{t,j} . k_s
        relu = np.maximum(dots, 0.0)                  # ReLU
        out[r, : p + 1] = np.asarray(w[i], dtype=np.float64) @ relu   # sum_j w_{t,j} * ...
    return out


def indexer_scores(q, k, w, q_scale=None, k_scale=None):
    """Full score tensor. q: [B, Lq, H, d], k: [B, Lk, d], w: [B, Lq, H];
    scales: [B, Lq] / [B, Lk] or None.  Returns [B, Lq, Lk] float64 (-inf where s > p_i)."""
    B, Lq = q.shape[0], q.shape[1]
    Lk = k.shape[1]
    out = np.empty((B, Lq, Lk))
    for b in range(B):
        out[b] = indexer_scores_rows(
            q[b], k[b], w[b], range(Lq), Lk,
            None if q_scale is None else q_scale[b],
            None if k_scale is None else k_scale[b], Lq)
    return out


# ---------------------------------------------------------------------------
# Top-k.  GLM-5.2 技术报告速览, section "IndexShare": keep the k highest-scoring keys
# (k = 2048 << L).  GLM-5 technical report, section 3.2: the operator must be
# deterministic.  Reading: ties go to the lower position, fewer than k causal keys
# select all of them, the result lists positions in ascending order and is padded
# with -1 to length k.
# ---------------------------------------------------------------------------

def topk_row(scores, n_valid, k):
    """Positions selected from scores[:n_valid]; returns int64 array of length k."""
    n = int(n_valid)
    out = np.full(k, -1, dtype=np.int64)
    if n <= 0:
        return out
    cand = np.asarray(scores[:n], dtype=np.float64)
    if n <= k:
        out[:n] = np.arange(n)
        return out
    # Rank by (-score, position): a stable sort of -score keeps equal scores in
    # position order, so the first k are the top-k with ties to the lower position.
    order = np.argsort(-cand, kind="stable")[:k]
    out[:] = np.sort(order)
    return out


def topk_rows(scores, n_valid, k):
    """scores: [R, N]; n_valid: [R] ints.  Returns [R, k] int64."""
    scores = np.asarray(scores)
    return np.stack([topk_row(scores[r], n_valid[r], k) for r in range(scores.shape[0])])


# ---------------------------------------------------------------------------
# Sparse core attention.  GLM 5.2: Built for Long Horizon Tasks, discussion section
# "DSA 与 IndexShare 的组合数据流": each layer reads the K/V of the selected positions
# from its own cache and recomputes score, softmax and value aggregation on them.
# Dense-masked form: logits over every key, -inf outside the selected set.
# MLA latent form (GLM-5 technical report section 2.1; same discussion section):
# K is the whole 576-d latent row (512-d compressed KV + 64-d RoPE key), V is its
# first 512 dims, and the query heads are already absorbed into 576-d.
# ---------------------------------------------------------------------------

def sparse_attention_rows(q, k, v, idx_rows, sm_scale, Hkv=1):
    """Attention of selected query rows of one sequence.

    q: [R, H, Dqk]; k: [Lk, Hkv, Dqk]; v: [Lk, Hkv, Dv]; idx_rows: [R, kk] (-1 = none).
    Query head h reads KV head h // (H // Hkv).
    Returns (out [R, H, Dv], lse [R, H]) with lse = log sum_{s in S} exp(logit_s)
    (natural log); a row with no selected key gives out = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    R, H, _ = q.shape
    Lk = k.shape[0]
    Dv = v.shape[2]
    group = H // Hkv
    out = np.zeros((R, H, Dv))
    lse = np.full((R, H), -np.inf)
    for r in range(R):
        sel = np.zeros(Lk, dtype=bool)
        ids = np.asarray(idx_rows[r])
        sel[ids[ids >= 0]] = True
        if not sel.any():
            continue
        for h in range(H):
            kh = h // group
            logits = sm_scale * (k[:, kh, :] @ q[r, h])          # every key (dense)
            logits = np.where(sel, logits, -np.inf)               # mask outside S_t
            m = logits.max()
            e = np.exp(logits - m)
            z = e.sum()
            out[r, h] = (e / z) @ v[:, kh, :]
            lse[r, h] = m + np.log(z)
    return out, lse


# ---------------------------------------------------------------------------
# IndexShare group.  GLM-5.2 技术报告速览, section "IndexShare": layers come in groups
# of 4 (1 Full + 3 Shared); the Full layer runs the indexer; the Shared layers reuse
# its index set and still run their own sparse attention.  GLM 5.2: Built for Long
# Horizon Tasks, section 5.2: Shared layers read their own KV cache at those positions.
# ---------------------------------------------------------------------------

def layer_group(full, layers, k, rows=None, all_full=None):
    """One IndexShare group for batch element 0..B-1.

    full: dict(q [B,Lq,H_I,d], k [B,Lk,d], w [B,Lq,H_I], q_scale, k_scale) decoded float64;
    layers: list of dict(q [B,Lq,H,Dqk], k [B,Lk,Hkv,Dqk], v [B,Lk,Hkv,Dv], sm_scale, Hkv);
    rows: query rows to evaluate (default all);
    all_full: optional list of per-layer indexer inputs (the all-Full comparator, where
    every layer runs its own indexer).
    Returns (idx [B,R,k] of the Full layer, [per-layer (out [B,R,H,Dv], lse [B,R,H])],
    per-layer idx [n_layers][B,R,k]).
    """
    B, Lq = full["q"].shape[0], full["q"].shape[1]
    Lk = full["k"].shape[1]
    rows = list(range(Lq)) if rows is None else list(rows)

    def select(ind):
        res = []
        for b in range(B):
            sc = indexer_scores_rows(
                ind["q"][b], ind["k"][b], ind["w"][b], rows, Lk,
                None if ind.get("q_scale") is None else ind["q_scale"][b],
                None if ind.get("k_scale") is None else ind["k_scale"][b], Lq)
            nv = [causal_position(Lq, Lk, i) + 1 for i in rows]
            res.append(topk_rows(sc, nv, k))
        return np.stack(res)

    idx_full = select(full)
    per_layer_idx = []
    outs = []
    for li, lay in enumerate(layers):
        idx_l = idx_full if all_full is None else select(all_full[li])
        per_layer_idx.append(idx_l)
        o_b, l_b = [], []
        for b in range(B):
            o, l = sparse_attention_rows(lay["q"][b][rows], lay["k"][b], lay["v"][b],
                                         idx_l[b], lay["sm_scale"], lay.get("Hkv", 1))
            o_b.append(o)
            l_b.append(l)
        outs.append((np.stack(o_b), np.stack(l_b)))
    return idx_full, outs, per_layer_idx
