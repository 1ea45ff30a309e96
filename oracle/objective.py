"""The group-centroid objective of the kept indexer and its gradient (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): used by the tests, never by the
product path.

GLM-5.2 技术报告速览 (mloasisblog), section "IndexShare": reusing one index set across
layers loses accuracy when each indexer was trained for its own layer only, so the kept
indexer is fit to the centroid of the attention distributions of the layers it serves,
pbar_t = (1 / (m + 1)) sum_{j=0..m} p_t^(l+j), with p_t^(l+j) the main attention
distribution of layer l + j averaged over its heads, aligned by KL.

Readings (the page gives the centroid and "KL" only):
* Sparse form: both distributions live on the query's selected set S_t (its index row);
  positions outside S_t carry no mass.
* The loss of row t is KL(pbar_t || pi_t), pi_t = softmax over S_t of the indexer scores
  I_t.  pbar is the target (no gradient reaches the attention).
* Gradients are taken with respect to the indexer operands q^I, w and k^I, with
  ReLU'(0) = 0; the gradient of the loss with respect to I_t is pi_t - pbar_t.
"""
import numpy as np


def _selected(idx_row):
    ids = np.asarray(idx_row)
    return np.nonzero(ids >= 0)[0], ids[ids >= 0]


def attention_centroid_rows(layers, idx_rows, rows):
    """pbar [R, kk] for query rows `rows` of one sequence, aligned with idx_rows [R, kk]
    (0 at -1 entries).  layers: list of dicts with q [Lq, H, Dqk], k [Lk, 1, Dqk] (the
    latent rows; keys are the whole row) and sm_scale; each layer's distribution is the
    mean over its H heads of softmax_{s in S_t}(sm_scale q[t, h] . k[s])."""
    idx_rows = np.asarray(idx_rows)
    out = np.zeros(idx_rows.shape)
    for lay in layers:
        q = np.asarray(lay["q"], dtype=np.float64)
        kk = np.asarray(lay["k"], dtype=np.float64)[:, 0, :]
        for r, t in enumerate(rows):
            slots, pos = _selected(idx_rows[r])
            if len(pos) == 0:
                continue
            logits = lay["sm_scale"] * (q[t] @ kk[pos].T)             # [H, n]
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            out[r, slots] += p.mean(axis=0) / len(layers)
    return out


def indexer_kl_rows(q, k, w, idx_rows, pbar, rows):
    """Loss and gradients of sum_r KL(pbar_r || pi_r) over query rows `rows` of one
    sequence.  q: [Lq, H_I, d] (decoded values), k: [Lk, d], w: [Lq, H_I], idx_rows and
    pbar: [R, kk].  Returns (loss [R], dq [R, H_I, d], dw [R, H_I], dk [Lk, d]); dk sums the
    contributions of the given rows."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    R = len(rows)
    H, d = q.shape[1], q.shape[2]
    loss = np.zeros(R)
    dq = np.zeros((R, H, d))
    dw = np.zeros((R, H))
    dk = np.zeros_like(k)
    for r, t in enumerate(rows):
        slots, pos = _selected(idx_rows[r])
        if len(pos) == 0:
            continue
        x = q[t] @ k[pos].T                                   # [H, n]
        relu = np.maximum(x, 0.0)
        score = w[t] @ relu                                   # I_t on S_t
        z = score - score.max()
        log_pi = z - np.log(np.exp(z).sum())
        pi = np.exp(log_pi)
        pb = np.asarray(pbar[r], dtype=np.float64)[slots]
        pos_mass = pb > 0
        loss[r] = np.sum(pb[pos_mass] * (np.log(pb[pos_mass]) - log_pi[pos_mass]))
        g = pi - pb                                           # d loss / d I_t
        dw[r] = relu @ g
        c = w[t][:, None] * (x > 0) * g[None, :]              # d loss / d x  [H, n]
        dq[r] = c @ k[pos]
        np.add.at(dk, pos, c.T @ q[t])
    return loss, dq, dw, dk
