"""Pins of the oracle's indexer score (CPU only).

The score is I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]) over causal s <= t
(GLM-5.2 技术报告速览, section "IndexShare", indexer-score equation).
"""
import numpy as np
import torch

import oracle
from oracle import indexer_scores, indexer_scores_rows

NEG = -np.inf


def _hand_case():
    # Worked by hand (derivation in the comments below).
    q = np.array([[[1, 2], [-1, 0]],
                  [[0, 1], [2, -1]],
                  [[1, 1], [1, -2]]], dtype=np.float64)[None]       # [1, 3, H=2, d=2]
    k = np.array([[1, 0], [0, 2], [-1, 1]], dtype=np.float64)[None]  # [1, 3, 2]
    w = np.array([[1, 2], [0.5, 1], [2, -1]], dtype=np.float64)[None]
    # t=0: s=0: h0 [1,2].[1,0]=1 -> 1*1; h1 [-1,0].[1,0]=-1 -> 0          => 1
    # t=1: s=0: h0 0 -> 0; h1 [2,-1].[1,0]=2 -> 1*2                         => 2
    #      s=1: h0 [0,1].[0,2]=2 -> 0.5*2; h1 [2,-1].[0,2]=-2 -> 0          => 1
    # t=2: s=0: h0 1 -> 2*1; h1 [1,-2].[1,0]=1 -> -1*1                      => 1
    #      s=1: h0 2 -> 2*2; h1 -4 -> 0                                      => 4
    #      s=2: h0 [1,1].[-1,1]=0 -> 0; h1 [1,-2].[-1,1]=-3 -> 0           => 0
    expected = np.array([[1, NEG, NEG], [2, 1, NEG], [1, 4, 0]], dtype=np.float64)[None]
    return q, k, w, expected


def test_hand_worked_example():
    q, k, w, expected = _hand_case()
    got = indexer_scores(q, k, w)
    assert np.array_equal(got, expected)


def test_relu_is_applied_per_head_before_weighting():
    # One head with a negative dot product and negative weight: ReLU must zero it
    # before the weight, so the score is 0, not +|w*x|.
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[-3.0, 0.0]]])
    w = np.array([[[-2.0]]])
    assert indexer_scores(q, k, w)[0, 0, 0] == 0.0


def test_nonnegative_dots_reduce_to_matmul():
    # With q, k >= 0 every dot product is >= 0, ReLU is the identity and, with H=1,
    # w=1, the score is the plain matrix product q k^T (a library routine), masked causally.
    rng = np.random.default_rng(1)
    L, d = 37, 5
    q = rng.random((1, L, 1, d))
    k = rng.random((1, L, d))
    w = np.ones((1, L, 1))
    got = indexer_scores(q, k, w)[0]
    ref = torch.matmul(torch.from_numpy(q[0, :, 0]), torch.from_numpy(k[0]).T).numpy()
    ref = np.where(np.tril(np.ones((L, L), dtype=bool)), ref, -np.inf)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=0)


def test_sign_and_homogeneity():
    rng = np.random.default_rng(2)
    B, L, H, d = 1, 29, 3, 4
    q = rng.standard_normal((B, L, H, d))
    k = rng.standard_normal((B, L, d))
    w = rng.random((B, L, H))
    I = indexer_scores(q, k, w)
    finite = np.isfinite(I)
    assert np.all(I[finite] >= 0)                         # w >= 0 -> I >= 0
    assert np.all(indexer_scores(q, k, -w)[finite] <= 0)  # sign flips with w
    # Positive homogeneity in one key row: scale k_s by alpha >= 0 -> column s scales.
    s, alpha = 7, 2.5
    k2 = k.copy(); k2[0, s] *= alpha
    I2 = indexer_scores(q, k2, w)
    np.testing.assert_allclose(I2[0, s:, s], alpha * I[0, s:, s], rtol=1e-13)
    other = [c for c in range(L) if c != s]
    assert np.array_equal(I2[0][:, other], I[0][:, other])
    # Scaling w by c > 0 scales every score by c.
    np.testing.assert_allclose(indexer_scores(q, k, 3.0 * w)[finite], 3.0 * I[finite], rtol=1e-13)


def test_head_permutation_invariance():
    rng = np.random.default_rng(3)
    B, L, H, d = 1, 23, 5, 3
    q = rng.standard_normal((B, L, H, d))
    k = rng.standard_normal((B, L, d))
    w = rng.random((B, L, H))
    perm = rng.permutation(H)
    np.testing.assert_allclose(indexer_scores(q[:, :, perm], k, w[:, :, perm]),
                               indexer_scores(q, k, w), rtol=1e-13)


def test_causality_and_query_offset():
    # With Lq < Lk the queries are the last Lq positions: query i sees p_i + 1 keys.
    rng = np.random.default_rng(4)
    Lq, Lk, H, d = 4, 10, 2, 3
    q = rng.standard_normal((Lq, H, d))
    k = rng.standard_normal((Lk, d))
    w = rng.random((Lq, H))
    I = indexer_scores_rows(q, k, w, range(Lq), Lk)
    for i in range(Lq):
        p = oracle.causal_position(Lq, Lk, i)
        assert p == Lk - Lq + i
        assert np.all(np.isfinite(I[i, : p + 1])) and np.all(np.isneginf(I[i, p + 1:]))
    # Changing keys beyond p_0 does not change row 0.
    k2 = k.copy(); k2[Lk - Lq + 1:] = 100.0
    I2 = indexer_scores_rows(q, k2, w, [0], Lk)
    assert np.array_equal(I2[0], I[0])


def test_fp8_scales_are_applied_to_the_dequantised_value():
    # q code 2 with scale 0.5 is the value 1; k code 3 with scale 2 is 6: score = w*1*6.
    q = np.array([[[[2.0]]]]); k = np.array([[[3.0]]]); w = np.array([[[0.25]]])
    got = indexer_scores(q, k, w, q_scale=np.array([[0.5]]), k_scale=np.array([[2.0]]))
    assert got[0, 0, 0] == 0.25 * 6.0


def test_integer_inputs_give_exact_integer_scores():
    rng = np.random.default_rng(5)
    B, L, H, d = 1, 40, 4, 8
    q = rng.integers(-4, 5, (B, L, H, d)).astype(np.float64)
    k = rng.integers(-4, 5, (B, L, d)).astype(np.float64)
    w = rng.integers(0, 3, (B, L, H)).astype(np.float64)
    I = indexer_scores(q, k, w)
    f = np.isfinite(I)
    assert np.array_equal(I[f], np.round(I[f]))
    # Integer-exact by construction: compare with an exact integer evaluation.
    qi, ki, wi = q.astype(np.int64), k.astype(np.int64), w.astype(np.int64)
    for t in range(L):
        dots = qi[0, t] @ ki[0, : t + 1].T
        exact = wi[0, t] @ np.maximum(dots, 0)
        assert np.array_equal(I[0, t, : t + 1], exact.astype(np.float64))


def _triple_loop_scores(q, k, w, Lk):
    """The indexer-score equation written out as plain Python loops over (query, key, head,
    dim), with the causal rule s <= p_i, p_i = Lk - Lq + i; keys past p_i get -inf."""
    Lq, H, d = len(q), len(q[0]), len(q[0][0])
    out = []
    for i in range(Lq):
        p = Lk - Lq + i
        row = []
        for s in range(Lk):
            if s > p:
                row.append(float("-inf"))
                continue
            total = 0.0
            for j in range(H):
                dot = 0.0
                for e in range(d):
                    dot += q[i][j][e] * k[s][e]
                total += w[i][j] * (dot if dot > 0.0 else 0.0)
            row.append(total)
        out.append(row)
    return out


def test_matches_triple_loop_on_tiny_inputs():
    # Brute force on tiny shapes, signed weights, and queries that are the last Lq of Lk
    # positions (so the causal offset is exercised); agreement to rtol 1e-12.
    rng = np.random.default_rng(11)
    for (Lq, Lk, H, d) in [(12, 12, 3, 4), (5, 9, 2, 3), (1, 7, 3, 4)]:
        q = rng.standard_normal((Lq, H, d))
        k = rng.standard_normal((Lk, d))
        w = rng.standard_normal((Lq, H))
        ref = np.array(_triple_loop_scores(q.tolist(), k.tolist(), w.tolist(), Lk))
        got = indexer_scores_rows(q, k, w, range(Lq), Lk)
        assert np.array_equal(np.isneginf(got), np.isneginf(ref))
        f = np.isfinite(ref)
        np.testing.assert_allclose(got[f], ref[f], rtol=1e-12, atol=1e-14)
        # the batched entry point agrees with the row form when Lq == Lk
        if Lq == Lk:
            full = indexer_scores(q[None], k[None], w[None])[0]
            assert np.array_equal(np.isneginf(full), np.isneginf(ref))
            np.testing.assert_allclose(full[f], ref[f], rtol=1e-12, atol=1e-14)
