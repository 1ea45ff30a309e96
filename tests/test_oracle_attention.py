"""Pins of the oracle's sparse attention and IndexShare group (CPU only)."""
import math

import numpy as np
import torch

import oracle
from oracle import sparse_attention_rows, layer_group, topk_rows, indexer_scores_rows


def test_hand_worked_two_keys():
    # logits 0 and ln 3 -> softmax (1/4, 3/4) -> out = 10/4 + 3*2/4 = 4, lse = ln 4.
    q = np.array([[[math.log(3.0)]]])                 # [R=1, H=1, D=1]
    k = np.array([[[0.0]], [[1.0]]])                  # [Lk=2, Hkv=1, 1]
    v = np.array([[[10.0]], [[2.0]]])
    out, lse = sparse_attention_rows(q, k, v, np.array([[0, 1]]), 1.0)
    assert abs(out[0, 0, 0] - 4.0) < 1e-14 and abs(lse[0, 0] - math.log(4.0)) < 1e-14
    out, lse = sparse_attention_rows(q, k, v, np.array([[1, -1]]), 1.0)
    assert out[0, 0, 0] == 2.0 and abs(lse[0, 0] - math.log(3.0)) < 1e-14
    out, lse = sparse_attention_rows(q, k, v, np.array([[-1, -1]]), 1.0)
    assert out[0, 0, 0] == 0.0 and np.isneginf(lse[0, 0])


def test_all_causal_keys_equals_dense_causal_sdpa():
    # k >= L: every causal key is selected, so the sparse attention is dense causal
    # softmax attention; compare with the library routine in float64.
    rng = np.random.default_rng(0)
    L, H, D, k = 24, 3, 8, 32
    q = rng.standard_normal((L, H, D)); kk = rng.standard_normal((L, H, D)); v = rng.standard_normal((L, H, D))
    scale = 1 / math.sqrt(D)
    idx = topk_rows(np.zeros((L, L)), np.arange(1, L + 1), k)
    out, _ = sparse_attention_rows(q, kk, v, idx, scale, Hkv=H)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(kk).permute(1, 0, 2),
        torch.from_numpy(v).permute(1, 0, 2), is_causal=True, scale=scale).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_single_key_returns_its_value_and_identical_rows():
    rng = np.random.default_rng(1)
    Lk, H, D, Dv = 16, 4, 6, 5
    q = rng.standard_normal((3, H, D)); k = rng.standard_normal((Lk, 1, D)); v = rng.standard_normal((Lk, 1, Dv))
    out, _ = sparse_attention_rows(q, k, v, np.array([[5], [0], [15]]), 0.3)
    for r, s in enumerate([5, 0, 15]):
        assert np.array_equal(out[r], np.broadcast_to(v[s, 0], (H, Dv)))
    v2 = np.broadcast_to(v[3], v.shape).copy()              # every row the same V
    out2, _ = sparse_attention_rows(q, k, v2, np.array([[1, 2, 9, -1]] * 3), 0.3)
    np.testing.assert_allclose(out2, np.broadcast_to(v[3, 0], out2.shape), rtol=1e-14)


def test_zero_query_averages_selected_values_and_gqa_mapping():
    rng = np.random.default_rng(2)
    Lk, H, Hkv, D = 12, 4, 2, 3
    k = rng.standard_normal((Lk, Hkv, D)); v = rng.standard_normal((Lk, Hkv, D))
    q = np.zeros((1, H, D))
    sel = np.array([[2, 5, 7]])
    out, lse = sparse_attention_rows(q, k, v, sel, 1.0, Hkv=Hkv)
    for h in range(H):
        np.testing.assert_allclose(out[0, h], v[[2, 5, 7], h // 2].mean(axis=0), rtol=1e-13)
        assert abs(lse[0, h] - math.log(3)) < 1e-14


def _small_group(seed=0, Lq=20, Lk=20, k=6, n_layers=4):
    rng = np.random.default_rng(seed)
    H_I, d_I, H, D = 3, 4, 2, 5
    full = {"q": rng.standard_normal((1, Lq, H_I, d_I)), "k": rng.standard_normal((1, Lk, d_I)),
            "w": rng.random((1, Lq, H_I))}
    layers = [{"q": rng.standard_normal((1, Lq, H, D)), "k": rng.standard_normal((1, Lk, 1, D)),
               "v": rng.standard_normal((1, Lk, 1, D)), "sm_scale": 0.4, "Hkv": 1}
              for _ in range(n_layers)]
    others = [{"q": rng.standard_normal((1, Lq, H_I, d_I)), "k": rng.standard_normal((1, Lk, d_I)),
               "w": rng.random((1, Lq, H_I))} for _ in range(n_layers)]
    return full, layers, others, k


def test_group_shared_layers_reuse_full_index_set():
    full, layers, _, k = _small_group()
    idx, outs, per_layer = layer_group(full, layers, k)
    for li in range(4):
        assert np.array_equal(per_layer[li], idx)            # Shared = Full's set, bitwise
        o, l = sparse_attention_rows(layers[li]["q"][0], layers[li]["k"][0], layers[li]["v"][0],
                                     idx[0], 0.4)
        assert np.array_equal(outs[li][0][0], o)             # standalone attention with idx_full
    # rows with t+1 <= k select every causal key
    for t in range(k):
        assert idx[0, t, : t + 1].tolist() == list(range(t + 1))


def test_group_all_full_comparator_uses_own_sets():
    full, layers, others, k = _small_group(seed=3)
    others[0] = full
    _, _, per_layer = layer_group(full, layers, k, all_full=others)
    idx_full, _, _ = layer_group(full, layers, k)
    assert np.array_equal(per_layer[0], idx_full)
    assert any(not np.array_equal(per_layer[i], idx_full) for i in range(1, 4))


def test_group_causality_perturbation():
    full, layers, _, k = _small_group(seed=4)
    idx, outs, _ = layer_group(full, layers, k, rows=[9])
    full2 = {kk: vv.copy() for kk, vv in full.items()}
    full2["k"][0, 10:] *= -7.0                                 # keys after position 9
    layers2 = [{kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in lay.items()}
               for lay in layers]
    for lay in layers2:
        lay["k"][0, 10:] = 50.0; lay["v"][0, 10:] = -50.0
    idx2, outs2, _ = layer_group(full2, layers2, k, rows=[9])
    assert np.array_equal(idx, idx2)
    for a, b in zip(outs, outs2):
        assert np.array_equal(a[0], b[0])


def test_group_selects_from_scores_of_the_full_layer():
    full, layers, _, k = _small_group(seed=5)
    idx, _, _ = layer_group(full, layers, k)
    sc = indexer_scores_rows(full["q"][0], full["k"][0], full["w"][0], range(20), 20)
    ref = topk_rows(sc, [oracle.causal_position(20, 20, i) + 1 for i in range(20)], k)
    assert np.array_equal(idx[0], ref)
