"""Pins of the oracle's group-centroid objective (CPU only): gradients against central
finite differences of the loss, the loss against its closed forms, and the centroid against
the (separately pinned) sparse-attention oracle."""
import numpy as np

from oracle import attention_centroid_rows, indexer_kl_rows, sparse_attention_rows


def _case(seed=0, Lq=4, Lk=9, H=3, d=5, kk=6):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Lq, H, d))
    k = rng.standard_normal((Lk, d))
    w = rng.standard_normal((Lq, H))
    rows = list(range(Lq))
    idx = np.full((Lq, kk), -1)
    pbar = np.zeros((Lq, kk))
    for t in rows:
        n = min(kk, Lk - Lq + t + 1) - (t % 2)              # some rows padded with -1
        idx[t, :n] = np.sort(rng.choice(Lk - Lq + t + 1, n, replace=False))
        p = rng.random(n) + 0.05
        pbar[t, :n] = p / p.sum()
    return q, k, w, idx, pbar, rows


def _loss(q, k, w, idx, pbar, rows):
    return indexer_kl_rows(q, k, w, idx, pbar, rows)[0].sum()


def test_gradients_match_central_differences():
    q, k, w, idx, pbar, rows = _case()
    _, dq, dw, dk = indexer_kl_rows(q, k, w, idx, pbar, rows)
    eps = 1e-6
    for name, arr, grad in (("q", q, dq), ("w", w, dw), ("k", k, dk)):
        num = np.zeros_like(arr)
        for ix in np.ndindex(arr.shape):
            a = arr.copy(); a[ix] += eps
            b = arr.copy(); b[ix] -= eps
            args = {"q": q, "k": k, "w": w}
            args[name] = a
            fa = _loss(args["q"], args["k"], args["w"], idx, pbar, rows)
            args[name] = b
            fb = _loss(args["q"], args["k"], args["w"], idx, pbar, rows)
            num[ix] = (fa - fb) / (2 * eps)
        np.testing.assert_allclose(grad.reshape(num.shape), num, rtol=1e-5, atol=1e-7, err_msg=name)


def test_loss_closed_forms():
    q, k, w, idx, pbar, rows = _case(seed=1)
    loss = indexer_kl_rows(q, k, w, idx, pbar, rows)[0]
    assert np.all(loss >= 0)
    for r, t in enumerate(rows):
        slots = np.nonzero(idx[r] >= 0)[0]
        pos = idx[r, slots]
        # the indexer's own distribution, by explicit loops
        score = [sum(w[t, j] * max(0.0, float(q[t, j] @ k[s])) for j in range(q.shape[1])) for s in pos]
        e = [np.exp(v - max(score)) for v in score]
        pi = np.array(e) / sum(e)
        # target = pi: zero loss and zero gradient
        own = np.zeros_like(pbar[r]); own[slots] = pi
        l0, dq0, dw0, _ = indexer_kl_rows(q, k, w, idx[r:r + 1], own[None], [t])
        assert abs(l0[0]) < 1e-12 and np.abs(dq0).max() < 1e-12 and np.abs(dw0).max() < 1e-12
        # one-hot target at slot i: loss = -log pi_i
        for i in range(len(slots)):
            hot = np.zeros_like(pbar[r]); hot[slots[i]] = 1.0
            li = indexer_kl_rows(q, k, w, idx[r:r + 1], hot[None], [t])[0][0]
            assert abs(li + np.log(pi[i])) < 1e-12
        # the general case: sum p log(p / pi)
        pb = pbar[r, slots]
        assert abs(loss[r] - float(np.sum(pb * np.log(pb / pi)))) < 1e-12


def test_centroid_against_the_attention_oracle():
    rng = np.random.default_rng(2)
    Lq, Lk, H, D, Dv, kk = 3, 11, 4, 12, 8, 5
    lay = {"q": rng.standard_normal((Lq, H, D)), "k": rng.standard_normal((Lk, 1, D)), "sm_scale": 0.3}
    idx = np.array([[0, 3, 5, 8, -1], [1, 2, 4, 6, 9], [10, -1, -1, -1, -1]])
    rows = [0, 1, 2]
    pbar = attention_centroid_rows([lay], idx, rows)
    assert np.all(pbar[idx < 0] == 0)
    np.testing.assert_allclose(pbar.sum(axis=1), 1.0, rtol=1e-12)
    assert pbar[2, 0] == 1.0                                  # a single selected key
    # sum_i pbar_i V[s_i] is the head mean of the attention output (V = first Dv dims)
    v = lay["k"][:, :, :Dv]
    out, _ = sparse_attention_rows(lay["q"], lay["k"], v, idx, lay["sm_scale"], Hkv=1)
    for r in rows:
        sel = idx[r] >= 0
        np.testing.assert_allclose(pbar[r, sel] @ v[idx[r, sel], 0], out[r].mean(axis=0), rtol=1e-12, atol=1e-12)
    # the centroid of a layer with itself is that layer; two layers average
    np.testing.assert_allclose(attention_centroid_rows([lay, lay], idx, rows), pbar, rtol=1e-12)
    lay2 = {"q": rng.standard_normal((Lq, H, D)), "k": rng.standard_normal((Lk, 1, D)), "sm_scale": 0.5}
    p2 = attention_centroid_rows([lay2], idx, rows)
    np.testing.assert_allclose(attention_centroid_rows([lay, lay2], idx, rows), (pbar + p2) / 2, rtol=1e-12)
