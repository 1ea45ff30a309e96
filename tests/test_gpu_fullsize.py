"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times,
checked against the fp64 oracle on sampled query rows (the oracle computes each sampled row
over all of its causal keys).

* prefill 16384 tokens, bf16 indexer, k = 2048, the attention of all four layers of the group;
* prefill 131072 tokens, FP8 indexer, k = 2048, MLA attention of a Full and a Shared layer;
* decode: 64 sequences x 200001 keys (1 query each) and the 4-query MTP variant sharing the
  first query's index row;
* the last 4096-query chunk of a 1,048,576-token prefill;
* chunked prefill (4096-query chunks) equals the unchunked call bit for bit.

Bars as in test_gpu_parity: index sets equal except inside the tau band around the row's
k-th oracle score (tau 1e-3 for bf16, 2e-2 for FP8); attention max|err| <= 1e-2 * RMS(oracle output) on the
kernel's fp32 result, and the bf16 output equal to the round-to-nearest-even of that result.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import dsa_lightning_indexer_scores_amd as dsa
from tests._helpers import to_f64, index_sets_agree, poisoned, all_written

pytestmark = pytest.mark.gpu

DEV = "cuda"
TAU_FP8 = 2e-2


def _say(*a):
    print("[fullsize]", *a, file=sys.stderr, flush=True)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _oracle_score_row(ind, b, r, Lq, Lk, kI=None, ks=None):
    """fp64 scores of query row r of sequence b (position Lk - Lq + r) over all keys."""
    p = Lk - Lq + r
    kI = to_f64(ind["k"][b]) if kI is None else kI
    ks = to_f64(ind["k_scale"][b]) if ks is None else ks
    q = to_f64(ind["q"][b, r:r + 1])
    w = to_f64(ind["w"][b, r:r + 1])
    qs = to_f64(ind["q_scale"][b, r:r + 1])
    # the single query passed as the last of (Lk - p) queries sits at position p
    return oracle.indexer_scores_rows(q, kI, w, [0], Lk, qs, ks, Lk - p)[0], p


def _check_sets(idx_rows, score_rows, positions, k):
    sc = np.stack(score_rows)
    nv = [p + 1 for p in positions]
    ref = oracle.topk_rows(sc, nv, k)
    ok, nbad, msg = index_sets_agree(idx_rows, ref, sc, nv, k, TAU_FP8)
    assert ok, msg
    return nbad


def _check_attention(q_rows, kv_rows, idx_rows, sm_scale, got32):
    """Oracle attention of the sampled rows.  kv_rows(j) gives (K, idx) for row j: the
    sequence's float64 latent rows [n, 576] and the row's index list into them (either the
    whole cache with the selected positions, or only the selected rows, which is the same
    definition restricted to the listed keys)."""
    refs = []
    for j in range(q_rows.shape[0]):
        kv, ir = kv_rows(j)
        ref, _ = oracle.sparse_attention_rows(q_rows[j:j + 1], kv[:, None, :], kv[:, None, :512],
                                              ir[None], sm_scale, 1)
        refs.append(ref[0])
    ref = np.stack(refs)
    rms = math.sqrt(float(np.mean(ref ** 2)))
    err = float(np.abs(got32 - ref).max())
    assert err <= 1e-2 * rms, (err, rms)
    return err / rms


def _poisoned(shape, dtype):
    return poisoned(shape, dtype, DEV)


def test_prefill128k_full_size_sampled_rows():
    cfg = synth.get_config("prefill128k")
    L, k = cfg.L, cfg.topk
    _say("prefill128k: generating indexer inputs")
    ind = synth.indexer_inputs(cfg, device=DEV)
    ws = dsa.Workspace()
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, q_scale=ind["q_scale"],
                           k_scale=ind["k_scale"], ws=ws, out=_poisoned((1, L, k), torch.int32))
    torch.cuda.synchronize()
    assert all_written(idx)
    rng = np.random.default_rng(11)
    rows = sorted(set([0, 1, k - 2, k - 1, k, L // 2, L - 2, L - 1] + rng.integers(0, L, 4).tolist()))
    _say("prefill128k: oracle scores of rows", rows)
    kI, ks = to_f64(ind["k"][0]), to_f64(ind["k_scale"][0])
    scs, pos = zip(*[_oracle_score_row(ind, 0, r, L, L, kI, ks) for r in rows])
    idx_np = idx[0, rows].cpu().numpy()
    nbad = _check_sets(idx_np, scs, pos, k)
    _say(f"prefill128k: index sets agree ({nbad} rows differ inside the band)")
    del ind, kI
    _free()
    for layer in (0, 3):                         # the Full layer and a Shared layer
        lay = synth.attention_inputs(cfg, layer=layer, device=DEV)
        out32 = dsa.sparse_attn(lay, idx, ws=ws, out=_poisoned((1, L, cfg.H, cfg.Dv), torch.float32))
        outbf = dsa.sparse_attn(lay, idx, ws=ws, out=_poisoned((1, L, cfg.H, cfg.Dv), torch.bfloat16))
        assert all_written(out32) and all_written(outbf)
        assert torch.equal(outbf, out32.to(torch.bfloat16))
        kv = to_f64(lay["kv"][0])
        rel = _check_attention(to_f64(lay["q"][0, rows]), lambda j: (kv, idx_np[j]), idx_np,
                               lay["sm_scale"], out32[0, rows].cpu().numpy().astype(np.float64))
        _say(f"prefill128k: layer {layer} attention max|err|/RMS = {rel:.2e}")
        del lay, out32, outbf, kv
        _free()


def test_prefill16k_full_size_group():
    """The 16384-token prefill with a bf16 indexer (H_I = 64, d_I = 128), k = 2048, and a
    4-layer group (1 Full + 3 Shared), in the benchmark's launch configuration: one fused
    indexer + top-k, then each layer's sparse attention with that index set.  Sampled rows
    against the oracle (index sets inside the bf16 band, attention of every layer), every
    output element written, and dsa_layer_group giving the same bits."""
    cfg = synth.get_config("prefill16k")
    L, k = cfg.L, cfg.topk
    _say("prefill16k: generating inputs")
    ind = synth.indexer_inputs(cfg, device=DEV)
    layers = [synth.attention_inputs(cfg, layer=l, device=DEV) for l in range(cfg.n_layers)]
    ws = dsa.Workspace()
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, ws=ws, out=_poisoned((1, L, k), torch.int32))
    outs32 = [dsa.sparse_attn(lay, idx, ws=ws, out=_poisoned((1, L, cfg.H, cfg.Dv), torch.float32))
              for lay in layers]
    outsbf = [dsa.sparse_attn(lay, idx, ws=ws, out=_poisoned((1, L, cfg.H, cfg.Dv), torch.bfloat16))
              for lay in layers]
    torch.cuda.synchronize()
    assert all_written(idx)
    for l in range(cfg.n_layers):
        assert all_written(outs32[l]) and all_written(outsbf[l]), f"layer {l}: unwritten output"
        assert torch.equal(outsbf[l], outs32[l].to(torch.bfloat16)), f"layer {l}: bf16 output is not RNE(fp32)"
    # the C-ABI group call gives the same index set and outputs
    gidx, gouts = dsa.layer_group(ind, layers, k, ws=ws, idx_out=_poisoned((1, L, k), torch.int32),
                                  outs=[_poisoned((1, L, cfg.H, cfg.Dv), torch.bfloat16) for _ in layers])
    assert torch.equal(gidx, idx)
    for l in range(cfg.n_layers):
        assert torch.equal(gouts[l], outsbf[l])
    rng = np.random.default_rng(16)
    rows = sorted(set([0, 1, k - 2, k - 1, k, L // 2, L - 2, L - 1] + rng.integers(0, L, 4).tolist()))
    _say("prefill16k: oracle scores of rows", rows)
    kI = to_f64(ind["k"][0])
    q = to_f64(ind["q"][0, rows])
    w = to_f64(ind["w"][0, rows])
    scs = [oracle.indexer_scores_rows(q[j:j + 1], kI, w[j:j + 1], [0], L, None, None, L - r)[0]
           for j, r in enumerate(rows)]
    idx_np = idx[0, rows].cpu().numpy()
    sc = np.stack(scs)
    nv = [r + 1 for r in rows]
    ref = oracle.topk_rows(sc, nv, k)
    ok, nbad, msg = index_sets_agree(idx_np, ref, sc, nv, k, 1e-3)
    assert ok, msg
    _say(f"prefill16k: index sets agree ({nbad} rows differ inside the band)")
    for l, lay in enumerate(layers):
        kv = to_f64(lay["kv"][0])
        rel = _check_attention(to_f64(lay["q"][0, rows]), lambda j: (kv, idx_np[j]), idx_np,
                               lay["sm_scale"], outs32[l][0, rows].cpu().numpy().astype(np.float64))
        _say(f"prefill16k: layer {l} attention max|err|/RMS = {rel:.2e}")


def _varlen_lengths(B, Lk):
    """Seeded cache lengths of a variable-length decode batch: uniform in [Lk/2, Lk]."""
    return np.random.default_rng(5).integers(Lk // 2, Lk + 1, B).astype(np.int32)


def test_decode200k_full_size_and_mtp():
    cfg = synth.get_config("decode200k")
    B, Lk, k = cfg.B, cfg.L, cfg.topk
    _say("decode200k: generating indexer inputs")
    ind = synth.indexer_inputs(cfg, device=DEV)
    ws = dsa.Workspace()
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, q_scale=ind["q_scale"],
                           k_scale=ind["k_scale"], ws=ws, out=_poisoned((B, 1, k), torch.int32))   # [B, 1, k]
    torch.cuda.synchronize()
    assert all_written(idx)
    seqs = [0, 17, B - 1]
    scs, pos = zip(*[_oracle_score_row(ind, b, 0, 1, Lk) for b in seqs])
    idx_np = idx[seqs, 0].cpu().numpy()
    nbad = _check_sets(idx_np, scs, pos, k)
    _say(f"decode200k: index sets of sequences {seqs} agree ({nbad} differ inside the band)")
    # the same caches as a variable-length batch (the decode launch of the benchmark's
    # varlen line): sequence b holds its first lens[b] keys; sampled sequences equal the
    # call on their own cache
    lens = torch.from_numpy(_varlen_lengths(B, Lk)).to(DEV)
    idx_v = dsa.indexer_topk_varlen(ind["q"], ind["k"], ind["w"], k, lens, q_scale=ind["q_scale"],
                                    k_scale=ind["k_scale"], ws=ws, out=_poisoned((B, 1, k), torch.int32))
    assert all_written(idx_v)
    for b in seqs:
        n = int(lens[b])
        ref = dsa.indexer_topk(ind["q"][b:b + 1], ind["k"][b:b + 1, :n], ind["w"][b:b + 1], k,
                               q_scale=ind["q_scale"][b:b + 1], k_scale=ind["k_scale"][b:b + 1, :n], ws=ws)
        assert torch.equal(idx_v[b], ref[0]), b
    _say(f"decode200k varlen: sequences {seqs} (lengths {[int(lens[b]) for b in seqs]}) equal their own calls")
    del ind
    _free()
    lay = synth.attention_inputs(cfg, layer=0, device=DEV)
    out32 = dsa.sparse_attn(lay, idx, ws=ws, out=_poisoned((B, 1, cfg.H, cfg.Dv), torch.float32))
    outbf = dsa.sparse_attn(lay, idx, ws=ws, out=_poisoned((B, 1, cfg.H, cfg.Dv), torch.bfloat16))
    assert all_written(out32) and all_written(outbf)
    assert torch.equal(outbf, out32.to(torch.bfloat16))
    for j, b in enumerate(seqs):
        kv = to_f64(lay["kv"][b])
        rel = _check_attention(to_f64(lay["q"][b, 0:1]), lambda _, j=j: (kv, idx_np[j]), idx_np[j:j + 1],
                               lay["sm_scale"], out32[b, 0:1].cpu().numpy().astype(np.float64))
        _say(f"decode200k: sequence {b} attention max|err|/RMS = {rel:.2e}")
    del lay, out32, outbf
    _free()
    # MTP draft: 4 queries per sequence share the first step's index row
    lay4 = synth.attention_inputs(cfg, layer=1, device=DEV, Lq=cfg.mtp)
    out4 = dsa.sparse_attn(lay4, idx, idx_q_stride=0, ws=ws, out=_poisoned((B, cfg.mtp, cfg.H, cfg.Dv), torch.float32))
    assert all_written(out4)
    for j, b in enumerate(seqs[:2]):
        kv = to_f64(lay4["kv"][b])
        rel = _check_attention(to_f64(lay4["q"][b]), lambda _, j=j: (kv, idx_np[j]),
                               np.repeat(idx_np[j:j + 1], cfg.mtp, axis=0),
                               lay4["sm_scale"], out4[b].cpu().numpy().astype(np.float64))
        _say(f"decode200k MTP: sequence {b} attention max|err|/RMS = {rel:.2e}")
    del lay4, out4
    _free()


def test_chunk1m_last_chunk_sampled_rows():
    cfg = synth.get_config("chunk1m")
    Lk, C, k = cfg.L, cfg.chunk, cfg.topk
    _say("chunk1m: generating the last chunk's indexer inputs")
    ind = synth.indexer_inputs(cfg, device=DEV, Lq=C)                 # queries Lk-C .. Lk-1
    ws = dsa.Workspace()
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, q_scale=ind["q_scale"],
                           k_scale=ind["k_scale"], ws=ws, out=_poisoned((1, C, k), torch.int32))
    torch.cuda.synchronize()
    assert all_written(idx)
    rng = np.random.default_rng(12)
    rows = sorted(set([0, 1, C // 2, C - 1] + rng.integers(0, C, 2).tolist()))
    kI, ks = to_f64(ind["k"][0]), to_f64(ind["k_scale"][0])
    scs, pos = zip(*[_oracle_score_row(ind, 0, r, C, Lk, kI, ks) for r in rows])
    idx_np = idx[0, rows].cpu().numpy()
    nbad = _check_sets(idx_np, scs, pos, k)
    _say(f"chunk1m: index sets of rows {rows} agree ({nbad} differ inside the band)")
    del ind, kI
    _free()
    lay = synth.attention_inputs(cfg, layer=0, device=DEV, Lq=C)
    out32 = dsa.sparse_attn(lay, idx, ws=ws, out=_poisoned((1, C, cfg.H, cfg.Dv), torch.float32))
    assert all_written(out32)

    def selected_rows(j):                        # only the listed rows of the 1M-row cache
        sel = idx_np[j][idx_np[j] >= 0]
        kv = to_f64(lay["kv"][0, torch.from_numpy(sel.astype(np.int64)).to(DEV)])
        return kv, np.arange(len(sel))

    rel = _check_attention(to_f64(lay["q"][0, rows]), selected_rows, idx_np, lay["sm_scale"],
                           out32[0, rows].cpu().numpy().astype(np.float64))
    _say(f"chunk1m: attention max|err|/RMS = {rel:.2e}")
    del lay, out32
    _free()


def test_chunked_prefill_equals_unchunked():
    L, C, k = 16384, 4096, 2048
    cfg = synth.get_config("chunk1m", L=L)
    ind = synth.indexer_inputs(cfg, device=DEV, Lq=L)
    full = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, q_scale=ind["q_scale"], k_scale=ind["k_scale"])
    for c in range(L // C):
        lo, hi = c * C, (c + 1) * C
        part = dsa.indexer_topk(ind["q"][:, lo:hi], ind["k"][:, :hi], ind["w"][:, lo:hi], k,
                                q_scale=ind["q_scale"][:, lo:hi], k_scale=ind["k_scale"][:, :hi])
        assert torch.equal(part, full[:, lo:hi]), f"chunk {c}"


def test_projections_full_size_sampled_rows():
    """The q^I map the bench times (4096 tokens, D = 6144, N = 64 x 128): sampled rows
    against the oracle's float64 dot products within the bound of K fp32 roundings."""
    T, D, N = 4096, 6144, 64 * 128
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    h = torch.randn((T, D), generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    wq = (torch.randn((N, D), generator=g, device=DEV, dtype=torch.float32) * D ** -0.5).to(torch.bfloat16)
    y = dsa.linear_bf16(h, wq)
    rows = [0, 1, 127, 128, 2047, 4095] + np.random.default_rng(3).integers(0, T, 4).tolist()
    xo, wo = to_f64(h[rows]), to_f64(wq)
    ref = oracle.linear(xo, wo)
    bound = D * 2.0 ** -24 * (np.abs(xo) @ np.abs(wo).T) * 1.01
    err = np.abs(y[rows].cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= bound), f"worst excess {np.max(err - bound)}"


def test_indexer_training_16k_sampled():
    """The training step the bench times (16K bf16, k = 2048, 4 MLA layers): the centroid,
    the loss, dq and dw on sampled rows, and dk on sampled keys (summed over every row that
    selected them), against the oracle with the bounds of the small-size parity test."""
    cfg = synth.get_config("prefill16k")
    ind = synth.indexer_inputs(cfg, device=DEV)
    layers = [synth.attention_inputs(cfg, layer=l, device=DEV) for l in range(cfg.n_layers)]
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], cfg.topk)
    lses = [dsa.sparse_attn(lay, idx, return_lse=True)[1] for lay in layers]
    pbar = dsa.attention_centroid(layers, idx, lses)
    out = dsa.indexer_kl_backward(ind["q"], ind["k"], ind["w"], idx, pbar)
    idx_h = idx[0].cpu().numpy()
    pb = pbar[0].cpu().numpy().astype(np.float64)
    rows = [0, 1, 2047, 2048, 9000, cfg.Lq - 1] + np.random.default_rng(4).integers(0, cfg.Lq, 3).tolist()
    # centroid on the sampled rows
    ora_layers = [{"q": to_f64(lay["q"][0, rows]), "k": to_f64(lay["kv"][0])[:, None, :], "sm_scale": lay["sm_scale"]}
                  for lay in layers]
    ref_p = oracle.attention_centroid_rows(ora_layers, idx_h[rows], list(range(len(rows))))
    np.testing.assert_allclose(pb[rows], ref_p, rtol=1e-4, atol=1e-7)
    # loss, dq, dw on the sampled rows (the GPU's centroid is the target of both sides)
    q = to_f64(ind["q"][0])
    kk = to_f64(ind["k"][0])
    w = to_f64(ind["w"][0])
    loss, dq, dw, _ = oracle.indexer_kl_rows(q, kk, w, idx_h[rows], pb[rows], rows)
    np.testing.assert_allclose(out["loss"][0, rows].cpu().numpy(), loss, rtol=1e-4, atol=1e-6)

    def bounds(t, r):
        sel = idx_h[t][idx_h[t] >= 0]
        x = q[t] @ kk[sel].T
        score = w[t] @ np.maximum(x, 0)
        pi = np.exp(score - score.max()); pi /= pi.sum()
        gg = pi - pb[t][idx_h[t] >= 0]
        dg = 1e-4 * pi + 1e-9
        tau = 2.0 ** -18 * (np.abs(q[t]) @ np.abs(kk[sel]).T)
        near = np.abs(x) <= tau
        c_err = 2.0 ** -8 * np.abs(w[t])[:, None] * ((x > 0) | near) * (np.abs(gg) + dg)[None, :] \
            + np.abs(w[t])[:, None] * ((x > 0) | near) * dg[None, :] + np.abs(w[t])[:, None] * near * np.abs(gg)[None, :]
        bw = (np.abs(x) * (dg[None, :] + 2.0 ** -16 * np.abs(gg)[None, :])).sum(axis=1) + (near * tau * np.abs(gg)[None, :]).sum(axis=1)
        return sel, c_err, bw

    got_dq = out["dq"][0, rows].cpu().numpy()
    got_dw = out["dw"][0, rows].cpu().numpy()
    for r, t in enumerate(rows):
        sel, c_err, bw = bounds(t, r)
        assert np.all(np.abs(got_dq[r] - dq[r]) <= c_err @ np.abs(kk[sel]) + 1e-6 * np.abs(dq).max()), f"dq row {t}"
        assert np.all(np.abs(got_dw[r] - dw[r]) <= bw + 1e-6 * np.abs(dw).max()), f"dw row {t}"
    # dk on sampled keys: every row that selected them contributes
    counts = np.bincount(idx_h[idx_h >= 0], minlength=cfg.L)
    used = np.nonzero(counts)[0]
    order = used[np.argsort(counts[used], kind="stable")]
    keys = [int(order[0]), int(order[len(order) // 2]), int(order[(3 * len(order)) // 4])]   # light to typical
    got_dk = out["dk"][0].cpu().numpy()
    for s in keys:
        src = np.nonzero((idx_h == s).any(axis=1))[0].tolist()
        if not src:
            continue
        _, _, _, dk = oracle.indexer_kl_rows(q, kk, w, idx_h[src], pb[src], src)
        lim = np.zeros(kk.shape[1])
        for t in src:
            sel, c_err, _ = bounds(t, 0)
            j = int(np.nonzero(sel == s)[0][0])
            lim += c_err[:, j] @ np.abs(q[t])
        assert np.all(np.abs(got_dk[s] - dk[s]) <= lim + 1e-6 * np.abs(dk[s]).max()), f"dk key {s} ({len(src)} rows)"
