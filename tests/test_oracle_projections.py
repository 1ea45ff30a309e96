"""Pins of the oracle's indexer projections (CPU only): the linear map against brute force,
closed forms and algebraic identities; the composed projections against the per-token
quantizer's definition."""
import numpy as np

from oracle import linear, indexer_projections, decode_e4m3


def test_linear_equals_brute_force_loops():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 7))
    w = rng.standard_normal((3, 7))
    ref = np.zeros((5, 3))
    for m in range(5):
        for n in range(3):
            acc = 0.0
            for k in range(7):
                acc += x[m, k] * w[n, k]
            ref[m, n] = acc
    np.testing.assert_allclose(linear(x, w), ref, rtol=1e-12, atol=1e-12)


def test_linear_closed_forms():
    rng = np.random.default_rng(1)
    w = rng.integers(-8, 9, (6, 4)).astype(np.float64)
    # one-hot rows pick a column of w: y[i, n] = w[n, i]
    np.testing.assert_array_equal(linear(np.eye(4), w), w.T)
    # w = identity returns x itself (a wrong transpose or index would not)
    x = rng.integers(-8, 9, (3, 4)).astype(np.float64)
    np.testing.assert_array_equal(linear(x, np.eye(4)), x)
    # a hand-worked case
    assert linear(np.array([[1.0, 2.0, 3.0]]), np.array([[4.0, 5.0, 6.0], [-1.0, 0.0, 1.0]])).tolist() == [[32.0, 2.0]]


def test_linear_identities():
    rng = np.random.default_rng(2)
    x1, x2 = rng.standard_normal((2, 4, 9))
    w = rng.standard_normal((5, 9))
    np.testing.assert_allclose(linear(2.0 * x1 - 3.0 * x2, w), 2.0 * linear(x1, w) - 3.0 * linear(x2, w), rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_allclose(linear(x1, w), linear(w, x1).T, rtol=0, atol=0)


def test_projections_quantize_each_token_of_the_linear_maps():
    rng = np.random.default_rng(3)
    T, D, H_I, d_I = 6, 64, 4, 8
    h = rng.standard_normal((T, D))
    h[2] = 0.0                                          # an all-zero token: scale 1, codes 0
    wq = rng.standard_normal((H_I * d_I, D))
    wk = rng.standard_normal((d_I, D))
    ww = rng.standard_normal((H_I, D))
    out = indexer_projections(h, wq, wk, ww, H_I)
    assert out["q"].shape == (T, H_I, d_I) and out["k"].shape == (T, d_I) and out["w"].shape == (T, H_I)
    assert out["q_scale"][2] == 1.0 and out["k_scale"][2] == 1.0
    assert not out["q"][2].any() and not out["k"][2].any()
    np.testing.assert_allclose(out["w"], h @ ww.T, rtol=1e-12)
    for name, wmat in (("q", wq), ("k", wk)):
        y = (h @ wmat.T).reshape(out[name].shape)
        s = out[name + "_scale"]
        # the scale is the token's amax / 448, and decoding gives y back to E4M3 precision
        # (relative 2^-4 for normal values, absolute 2^-10 scale for subnormals)
        amax = np.abs(y.reshape(T, -1)).max(axis=1)
        nz = amax > 0
        np.testing.assert_allclose(s[nz], (amax[nz] / 448.0).astype(np.float32), rtol=1e-7)
        back = decode_e4m3(out[name]) * s.reshape((T,) + (1,) * (y.ndim - 1))
        err = np.abs(back - y)
        bound = np.maximum(np.abs(y) * 2.0 ** -4, s.reshape((T,) + (1,) * (y.ndim - 1)) * 2.0 ** -10) * 1.0001
        assert np.all(err <= bound)
        # the largest value of each non-zero token is exactly +-448 in code space
        assert np.all(np.abs(decode_e4m3(out[name]).reshape(T, -1)).max(axis=1)[nz] == 448.0)
