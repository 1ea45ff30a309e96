"""The step before the path: the indexer's own projections (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): used by the tests, never by the
product path.

GLM 5.2: Built for Long Horizon Tasks (papers.chlience.com), discussion section
"DSA 与 IndexShare 的组合数据流": the indexer has its own light projections W_Q^I / W_K^I
and a per-layer index-key cache, beside the MLA path; the GLM-5.2 IndexShare page
(mloasisblog), section "IndexShare": the per-head gating weights w^I_{t,j}.  The pages give
neither the input of the projections nor their widths; the reading taken here is three
linear maps of the layer's hidden state h (q^I = h W_Q, k^I = h W_K, w = h W_w, weights in
the [out, in] layout of a linear layer), q^I and k^I then quantized per token to E4M3
exactly as ``formats.quantize_e4m3_per_token`` defines.
"""
import numpy as np

from .formats import quantize_e4m3_per_token


def linear(x, w):
    """y[m, n] = sum_k x[m, k] w[n, k] in float64 (x [M, K], w [N, K])."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def indexer_projections(h, wq, wk, ww, H_I):
    """Hidden states h [T, D] -> dict(q codes [T, H_I, d_I], q_scale [T], k codes [T, d_I],
    k_scale [T], w [T, H_I]) from y = linear(h, W) for each weight, the q^I / k^I rows
    quantized per token from their float32 values."""
    T = np.asarray(h).shape[0]
    d_I = np.asarray(wk).shape[0]
    yq = linear(h, wq).astype(np.float32).reshape(T, H_I, d_I)
    yk = linear(h, wk).astype(np.float32)
    q, q_scale = quantize_e4m3_per_token(yq)
    k, k_scale = quantize_e4m3_per_token(yk)
    return {"q": q, "q_scale": q_scale, "k": k, "k_scale": k_scale, "w": linear(h, ww)}
