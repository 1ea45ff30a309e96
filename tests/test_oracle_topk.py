"""Pins of the oracle's deterministic top-k (CPU only).

Reading of the pages: the k highest scores among the causal keys, ties to the lower
position, fewer than k candidates -> all of them, ascending positions, -1 padding.
"""
import numpy as np
import pytest

from oracle import topk_row, topk_rows


def test_hand_examples_with_ties():
    s = np.array([3.0, 1.0, 3.0, 2.0, 3.0])
    assert topk_row(s, 5, 2).tolist() == [0, 2]            # three 3's: the two lowest
    assert topk_row(s, 5, 4).tolist() == [0, 2, 3, 4]
    assert topk_row(s, 5, 1).tolist() == [0]
    assert topk_row(s, 4, 3).tolist() == [0, 2, 3]         # only the first 4 are causal
    assert topk_row(s, 2, 4).tolist() == [0, 1, -1, -1]    # fewer than k: all + padding
    assert topk_row(s, 0, 3).tolist() == [-1, -1, -1]


def test_signed_zero_ties():
    s = np.array([-0.0, 0.0, -0.0, -1.0])
    assert topk_row(s, 4, 2).tolist() == [0, 1]


def test_k1_is_first_argmax():
    rng = np.random.default_rng(0)
    for _ in range(50):
        s = rng.integers(0, 5, 30).astype(np.float64)        # many ties
        n = int(rng.integers(1, 31))
        assert topk_row(s, n, 1)[0] == int(np.argmax(s[:n]))   # numpy: first maximum


def _rank_definition(s, n, k):
    # Independent route: position j is selected iff fewer than k causal positions beat
    # it, where i beats j when s_i > s_j, or s_i == s_j and i < j.
    sel = []
    for j in range(n):
        beaten_by = sum(1 for i in range(n) if s[i] > s[j] or (s[i] == s[j] and i < j))
        if beaten_by < k:
            sel.append(j)
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("seed", range(6))
def test_matches_rank_definition(seed):
    rng = np.random.default_rng(seed)
    n_total = 60
    s = rng.integers(-3, 4, n_total).astype(np.float64) if seed % 2 else rng.standard_normal(n_total)
    for n in (1, 7, 33, 60):
        for k in (1, 5, 16, 59, 64):
            assert topk_row(s, n, k).tolist() == _rank_definition(s, n, k)


def test_lexsort_route_and_properties():
    rng = np.random.default_rng(7)
    R, N, k = 20, 300, 32
    s = rng.integers(0, 40, (R, N)).astype(np.float64)
    nv = rng.integers(1, N + 1, R)
    got = topk_rows(s, nv, k)
    for r in range(R):
        n = nv[r]
        order = np.lexsort((np.arange(n), -s[r, :n]))[:k]      # primary -score, then position
        ref = np.sort(order)
        row = got[r]
        assert row[: len(ref)].tolist() == ref.tolist()
        assert np.all(row[len(ref):] == -1)
        valid = row[row >= 0]
        assert np.all(np.diff(valid) > 0)                       # ascending
        assert len(valid) == min(k, n)
    assert np.array_equal(got, topk_rows(s, nv, k))             # run twice: identical


def test_rows_shorter_than_k_select_every_causal_key():
    rng = np.random.default_rng(8)
    s = rng.standard_normal((10, 50))
    k = 16
    nv = np.arange(1, 11)
    got = topk_rows(s, nv, k)
    for r in range(10):
        assert got[r, : nv[r]].tolist() == list(range(nv[r]))
        assert np.all(got[r, nv[r]:] == -1)
