"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bars (each derived where it is used, from the arithmetic of the kernel it checks):
* dsa_topk fed the oracle's fp32 scores: bit-exact (same idx array, order, padding).
* materialised scores: an element bound from the arithmetic (exact operand products,
  accumulation error of each dot product and of the head-weighted sum; see EPS_DOT).
* fused indexer + top-k: bit-identical to dsa_topk(dsa_indexer_scores) (same score
  bits), and index sets equal to the oracle's except for positions whose oracle score
  lies within tau*|theta| of the row's k-th score (tau 1e-3 bf16, 2e-2 fp8), sizes exact.
* sparse attention: max |err| <= 1e-2 * RMS(oracle output) with the GPU's idx.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import decode_e4m3
import synth
import dsa_lightning_indexer_scores_amd as dsa
from tests._helpers import to_f64, indexer_to_oracle, attn_to_oracle, index_sets_agree, poisoned, all_written

pytestmark = pytest.mark.gpu

DEV = "cuda"
TAU = {"bf16": 1e-3, "fp8": 2e-2, "f32": 1e-5}


def _cfg(dtype, L, k, **kw):
    base = "prefill16k" if dtype == "bf16" else ("prefill128k" if dtype == "fp8" else "tiny")
    return synth.get_config(base, L=L, Lq=kw.pop("Lq", L), topk=k, **kw)


def _ind_args(ind):
    return dict(q_scale=ind["q_scale"], k_scale=ind["k_scale"])


def _oracle_rows(ora, b, rows, Lq, Lk):
    return oracle.indexer_scores_rows(
        ora["q"][b], ora["k"][b], ora["w"][b], rows, Lk,
        None if ora["q_scale"] is None else ora["q_scale"][b],
        None if ora["k_scale"] is None else ora["k_scale"][b], Lq)


# ---------------------------------------------------------------------------
# top-k on the oracle's fp32 scores: bit-exact
# ---------------------------------------------------------------------------

def test_topk_bitexact_on_oracle_scores_tiny():
    cfg = synth.get_config("tiny")
    ind = synth.indexer_inputs(cfg, device="cpu")
    ora = indexer_to_oracle(ind)
    sc64 = oracle.indexer_scores(ora["q"], ora["k"], ora["w"])[0]        # [L, L]
    sc32 = sc64.astype(np.float32)
    L, k = cfg.L, cfg.topk
    n_valid = np.arange(1, L + 1, dtype=np.int32)
    ref = oracle.topk_rows(sc32.astype(np.float64), n_valid, k)
    got = dsa.topk(torch.from_numpy(sc32).to(DEV), k,
                   n_valid=torch.from_numpy(n_valid).to(DEV)).cpu().numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("case", ["gauss", "ties", "signed_zero", "k1", "k_ge_n", "long"])
def test_topk_bitexact_edge_cases(case):
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    if case == "gauss":
        rows, n, k = 37, 5003, 2048
        x = rng.standard_normal((rows, n)).astype(np.float32)
        nv = rng.integers(1, n + 1, rows).astype(np.int32)
        nv[:3] = [1, 2047, 2049]
    elif case == "ties":
        rows, n, k = 16, 3001, 100
        x = rng.integers(0, 4, (rows, n)).astype(np.float32)
        nv = np.full(rows, n, dtype=np.int32)
    elif case == "signed_zero":
        rows, n, k = 8, 700, 300
        x = rng.choice(np.array([0.0, -0.0, -1.0, 1.0, -2.5], dtype=np.float32), (rows, n))
        nv = np.full(rows, n, dtype=np.int32)
    elif case == "k1":
        rows, n, k = 9, 1000, 1
        x = rng.integers(0, 3, (rows, n)).astype(np.float32)
        nv = rng.integers(1, n + 1, rows).astype(np.int32)
    elif case == "k_ge_n":
        rows, n, k = 5, 300, 512
        x = rng.standard_normal((rows, n)).astype(np.float32)
        nv = np.array([300, 1, 299, 17, 0], dtype=np.int32)
    else:
        rows, n, k = 2, 200001, 2048
        x = (rng.standard_normal((rows, n)) * 3).astype(np.float32)
        nv = np.array([n, 150000], dtype=np.int32)
    ref = oracle.topk_rows(x.astype(np.float64), nv, k)
    # one workgroup per row, then (with a workspace) rows split over several workgroups
    for ws in (None, dsa.Workspace()):
        got_idx, got_val = dsa.topk(torch.from_numpy(x).to(DEV), k, n_valid=torch.from_numpy(nv).to(DEV),
                                    return_vals=True, ws=ws)
        got_idx = got_idx.cpu().numpy()
        assert np.array_equal(got_idx, ref)
        gv = got_val.cpu().numpy()
        for r in range(rows):
            sel = ref[r] >= 0
            assert np.array_equal(gv[r][sel], x[r][ref[r][sel]])
            assert np.all(np.isneginf(gv[r][~sel]))


@pytest.mark.parametrize("k,n,rows", [(8192, 30011, 3), (16384, 70001, 2), (65536, 100003, 2)])
def test_topk_bitexact_large_k(k, n, rows):
    # k above the on-chip list capacity: the selection runs over candidate lists in global
    # memory.  Heavy ties (values on a coarse grid) and rows with fewer than k candidates
    # are included; every idx and value element is written (outputs start poisoned).
    rng = np.random.default_rng(k + n)
    x = (rng.integers(-3000, 3000, (rows, n)) / 64.0).astype(np.float32)
    nv = np.array([n, k - 5] + [n // 2 + 7] * (rows - 2), dtype=np.int32)[:rows]
    ref = oracle.topk_rows(x.astype(np.float64), nv, k)
    for ws in (None, dsa.Workspace()):
        got_idx, got_val = dsa.topk(torch.from_numpy(x).to(DEV), k, n_valid=torch.from_numpy(nv).to(DEV),
                                    return_vals=True, ws=ws)
        assert np.array_equal(got_idx.cpu().numpy(), ref)
        gv = got_val.cpu().numpy()
        for r in range(rows):
            sel = ref[r] >= 0
            assert np.array_equal(gv[r][sel], x[r][ref[r][sel]])
            assert np.all(np.isneginf(gv[r][~sel]))


# ---------------------------------------------------------------------------
# materialised scores
# ---------------------------------------------------------------------------

# Element bound of the materialised scores.  The operand products are exact in fp32 (bf16
# and E4M3 significands are short), so the error is the accumulation of the d_I products
# of each dot product x_j (at most EPS_DOT times the sum of their magnitudes), passed
# through the 1-Lipschitz ReLU and weighted by |w_j|, plus the fp32 roundings of the
# head-weighted sum and the scale products (at most EPS_SUM = 2^-17 of sum_j |w_j x_j|,
# which covers 64 fused multiply-adds and two scale multiplications at 2^-24 each).
# EPS_DOT is the bound of a sequential fp32 sum of the d_I products: d_I * 2^-24, i.e.
# 2^-19 for the fp32 reference path (d_I = 32) and 2^-17 for bf16 and E4M3 (d_I = 128,
# summed by the matrix cores; their errors stay well inside it).
EPS_DOT = {"f32": 2.0 ** -19, "bf16": 2.0 ** -17, "fp8": 2.0 ** -17}
EPS_SUM = 2.0 ** -17


def _score_bounds(ora, b, rows, Lq, Lk):
    """Per-element error bound of the materialised scores of the given rows (see EPS_DOT)."""
    q = ora["q"][b]
    k = ora["k"][b]
    qs = None if ora["q_scale"] is None else ora["q_scale"][b]
    ks = None if ora["k_scale"] is None else ora["k_scale"][b]
    kk = k if ks is None else k * ks[:, None]
    out = np.zeros((len(rows), Lk))
    for r, i in enumerate(rows):
        qi = q[i] if qs is None else q[i] * qs[i]
        w = np.abs(ora["w"][b][i])
        absdot = np.abs(qi) @ np.abs(kk).T              # [H, Lk]  sum_d |q_jd k_sd|
        x = np.abs(qi @ kk.T)                           # [H, Lk]  |x_j|
        out[r] = EPS_DOT[ora["dtype"]] * (w @ absdot) + EPS_SUM * (w @ x)
    return out


@pytest.mark.parametrize("dtype,L,Lq,B", [("f32", 1024, 1024, 1), ("bf16", 600, 600, 1),
                                          ("fp8", 520, 520, 1), ("fp8", 5000, 3, 2), ("bf16", 777, 5, 2)])
def test_indexer_scores_parity(dtype, L, Lq, B):
    cfg = _cfg(dtype, L, 64, Lq=Lq, B=B)
    ind = synth.indexer_inputs(cfg, device=DEV)
    got = dsa.indexer_scores(ind["q"], ind["k"], ind["w"], **_ind_args(ind),
                             out=poisoned((B, Lq, L), torch.float32))
    assert all_written(got)
    got = got.cpu().numpy()
    ora = indexer_to_oracle(ind)
    ora["dtype"] = dtype
    rng = np.random.default_rng(0)
    rows = sorted(set([0, 1, Lq - 1] + rng.integers(0, Lq, 12).tolist()))
    worst = 0.0
    for b in range(B):
        ref = _oracle_rows(ora, b, rows, Lq, L)
        g = got[b][rows].astype(np.float64)
        assert np.array_equal(np.isneginf(g), np.isneginf(ref))
        fin = np.isfinite(ref)
        bound = _score_bounds(ora, b, rows, Lq, L)
        err = np.abs(np.where(fin, g, 0) - np.where(fin, ref, 0))
        ratio = err / (bound + 1e-30)
        worst = max(worst, float(ratio[fin].max()))
        assert np.all(err[fin] <= bound[fin]), (dtype, float(ratio[fin].max()))
    print(f"[scores] {dtype}: worst error / element bound = {worst:.3f}")



# Indexer head counts below 64 (one, two and three 16-head blocks; the bf16 score schedule
# pairs dot products, and with an odd count a pair spans two key blocks): materialised
# scores within the element bound, the fused index sets against the oracle's exact top-k
# within the tolerance band, and the fused kernel equal to the top-k of the materialised
# scores.  Prefill rows and a few-query (chunk list) call.
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("H_I", [16, 32, 48])
@pytest.mark.parametrize("Lq,Lk", [(700, 700), (2, 20000)])
def test_indexer_fewer_heads(dtype, H_I, Lq, Lk):
    k = 128
    cfg = _cfg(dtype, Lk, k, Lq=Lq, B=1, H_I=H_I)
    ind = synth.indexer_inputs(cfg, device=DEV)
    sc = dsa.indexer_scores(ind["q"], ind["k"], ind["w"], **_ind_args(ind))
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, **_ind_args(ind))
    nv = torch.arange(Lq, device=DEV, dtype=torch.int32) + (Lk - Lq + 1)
    assert torch.equal(idx[0], dsa.topk(sc[0], k, n_valid=nv))
    ora = indexer_to_oracle(ind)
    ora["dtype"] = dtype
    rows = sorted({0, Lq // 2, Lq - 1})
    ref = _oracle_rows(ora, 0, rows, Lq, Lk)
    g = sc[0].cpu().numpy()[rows].astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(g), np.isneginf(ref))
    bound = _score_bounds(ora, 0, rows, Lq, Lk)
    assert np.all(np.abs(g[fin] - ref[fin]) <= bound[fin])
    nvr = [Lk - Lq + r + 1 for r in rows]
    ok, _, msg = index_sets_agree(idx.cpu().numpy()[0][rows], oracle.topk_rows(ref, nvr, k), ref, nvr, k,
                                  1e-3 if dtype == "bf16" else 2e-2)
    assert ok, msg

# ---------------------------------------------------------------------------
# fused indexer + top-k
# ---------------------------------------------------------------------------

FUSED_CASES = [
    # dtype, B, Lq, Lk, k
    ("bf16", 1, 2048, 2048, 256),      # many compactions per row
    ("fp8", 1, 2048, 2048, 256),
    ("fp8", 1, 1000, 1000, 2048),      # every row shorter than k: all causal keys
    ("bf16", 2, 333, 333, 64),         # ragged tail, batch
    ("fp8", 2, 64, 32768, 512),        # few queries, long keys: key segments + merge
    ("bf16", 1, 48, 20000, 1),         # k = 1
    # fewer than 16 queries (decode): per-chunk candidate lists, then the row selection
    ("fp8", 3, 1, 50000, 2048),
    ("bf16", 2, 4, 9000, 512),
    ("fp8", 2, 15, 3000, 2048),        # rows shorter and longer than k
    ("fp8", 1, 1, 100, 64),            # one chunk
    # more work items than persistent workgroups; long rows start from a speculative
    # threshold estimated from a sample of the item's keys
    ("fp8", 1, 20000, 20000, 256),
    ("bf16", 1, 12000, 12000, 512),
    ("fp8", 1, 2048, 65536, 256),      # 8 key segments, 2048 items: checked by the merge
    ("fp8", 1, 9000, 9000, 1),         # k = 1: the sampled threshold sits near the sample's top
    ("bf16", 1, 12000, 12000, 4096),   # the largest k: the threshold deep in the sample
]


@pytest.mark.parametrize("dtype,B,Lq,Lk,k", FUSED_CASES)
def test_fused_topk_equals_scores_then_topk(dtype, B, Lq, Lk, k):
    cfg = _cfg(dtype, Lk, k, Lq=Lq, B=B)
    ind = synth.indexer_inputs(cfg, device=DEV)
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, **_ind_args(ind))
    sc = dsa.indexer_scores(ind["q"], ind["k"], ind["w"], **_ind_args(ind))
    nv = (torch.arange(Lq, device=DEV, dtype=torch.int32) + (Lk - Lq + 1)).repeat(B)
    ref = dsa.topk(sc.reshape(B * Lq, Lk), k, n_valid=nv).reshape(B, Lq, k)
    assert torch.equal(idx, ref)
    idx2 = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, **_ind_args(ind))
    assert torch.equal(idx, idx2)                                     # run twice: identical


@pytest.mark.parametrize("dtype,Lq,L,k", [("fp8", 20000, 20000, 256), ("bf16", 12000, 12000, 256),
                                          ("fp8", 2048, 65536, 2048)])
def test_fused_topk_speculation_failures_are_recomputed(dtype, Lq, L, k):
    """About one 64-key block in 64 gets a score scale of 100.  The rows hold too few such
    hot keys to fill their top k, so an item whose sample tiles meet a hot block starts its
    rows from a threshold far above their k-th score: they admit fewer than k keys and the
    second pass recomputes the item (with key segments the merge finds the failing rows).
    The launch must have recorded failures (the workspace's third int32 counts them), and
    the result must still equal dsa_topk(dsa_indexer_scores) bit for bit."""
    cfg = _cfg(dtype, L, k, Lq=Lq, B=1)
    ind = synth.indexer_inputs(cfg, device=DEV)
    rng = np.random.default_rng(13)
    hot = np.repeat(np.where(rng.random(L // 64 + 1) < 1 / 64, 100.0, 1.0), 64)[:L].astype(np.float32)
    f = torch.from_numpy(hot).to(DEV)
    if dtype == "fp8":
        ind["k_scale"] = (ind["k_scale"] * f[None]).contiguous()
    else:
        ind["k"] = (ind["k"].float() * f[None, :, None]).to(torch.bfloat16).contiguous()
    ws = dsa.Workspace()
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, ws=ws, **_ind_args(ind))
    fails = int(ws.buf[8:12].view(torch.int32).item())
    sc = dsa.indexer_scores(ind["q"], ind["k"], ind["w"], **_ind_args(ind))
    nv = torch.arange(L - Lq + 1, L + 1, device=DEV, dtype=torch.int32)
    assert torch.equal(idx, dsa.topk(sc.reshape(Lq, L), k, n_valid=nv).reshape(1, Lq, k))
    assert fails > 0


@pytest.mark.parametrize("dtype,B,Lq,Lk,k", FUSED_CASES[:5] + FUSED_CASES[6:7])
def test_fused_topk_matches_oracle_sets(dtype, B, Lq, Lk, k):
    cfg = _cfg(dtype, Lk, k, Lq=Lq, B=B)
    ind = synth.indexer_inputs(cfg, device=DEV)
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, **_ind_args(ind)).cpu().numpy()
    ora = indexer_to_oracle(ind)
    rng = np.random.default_rng(1)
    rows = sorted(set([0, min(k, Lq) - 1, min(k, Lq - 1), Lq - 1] + rng.integers(0, Lq, 10).tolist()))
    for b in range(B):
        sc = _oracle_rows(ora, b, rows, Lq, Lk)
        nv = [Lk - Lq + r + 1 for r in rows]
        ref = oracle.topk_rows(sc, nv, k)
        ok, nbad, msg = index_sets_agree(idx[b][rows], ref, sc, nv, k, TAU[dtype])
        assert ok, msg


@pytest.mark.parametrize("Lq", [1, 3])
def test_few_query_topk_heavy_ties_integer_exact(Lq):
    """Integer-exact E4M3 inputs: every head's query is e_0, key s is v_s e_0 with v_s in
    {1, 2}, w = 1/64, unit scales, so every score is exactly v_s.  Half the keys tie at
    the top: the k-th digit's bin overflows the LDS list and the selection runs over the
    chunk lists in global memory; ties go to the lower positions."""
    B, Lk, k, H, D = 2, 40000, 2048, 64, 128
    rng = np.random.default_rng(11)
    q = np.zeros((B, Lq, H, D), np.uint8)
    q[..., 0] = 0x38                                   # E4M3 1.0
    kk = np.zeros((B, Lk, D), np.uint8)
    kk[..., 0] = np.where(rng.random((B, Lk)) < 0.5, 0x40, 0x38)    # 2.0 or 1.0
    ind = {"q": torch.from_numpy(q).to(DEV), "k": torch.from_numpy(kk).to(DEV),
           "w": torch.full((B, Lq, H), 1.0 / 64, dtype=torch.float32, device=DEV),
           "q_scale": torch.ones((B, Lq), dtype=torch.float32, device=DEV),
           "k_scale": torch.ones((B, Lk), dtype=torch.float32, device=DEV), "dtype": "fp8", "H_I": H, "d_I": D}
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, **_ind_args(ind))
    sc = dsa.indexer_scores(ind["q"], ind["k"], ind["w"], **_ind_args(ind))
    nv = (torch.arange(Lq, device=DEV, dtype=torch.int32) + (Lk - Lq + 1)).repeat(B)
    assert torch.equal(idx, dsa.topk(sc.reshape(B * Lq, Lk), k, n_valid=nv).reshape(B, Lq, k))
    got = idx.cpu().numpy()
    ora = indexer_to_oracle(ind)
    for b in range(B):
        rows = list(range(Lq))
        osc = _oracle_rows(ora, b, rows, Lq, Lk)
        assert set(np.unique(osc[np.isfinite(osc)])) <= {1.0, 2.0}
        ref = oracle.topk_rows(osc, [Lk - Lq + r + 1 for r in rows], k)
        assert np.array_equal(got[b], ref)
        assert np.array_equal(got[b][0], np.flatnonzero(kk[b, :, 0] == 0x40)[:k])


@pytest.mark.parametrize("dtype,Lq,k", [("fp8", 1, 2048), ("bf16", 4, 512), ("fp8", 3, 64)])
def test_varlen_decode_equals_each_sequence_alone(dtype, Lq, k):
    """A decode batch whose caches hold different numbers of keys: each sequence's index
    rows equal dsa_indexer_topk on that sequence's own cache (bit-exact).  Lengths include
    the full cache, one key, no key, fewer than Lq keys, fewer and a few more than k."""
    B, Lmax = 7, 30000
    cfg = _cfg(dtype, Lmax, k, Lq=Lq, B=B)
    ind = synth.indexer_inputs(cfg, device=DEV)
    lens_l = [Lmax, 1, 0, max(Lq - 1, 0), k // 2, k + 5, 17777]
    lens = torch.tensor(lens_l, dtype=torch.int32, device=DEV)
    idx = dsa.indexer_topk_varlen(ind["q"], ind["k"], ind["w"], k, lens, **_ind_args(ind))
    got = idx.cpu().numpy()
    sc = lambda t, b, n: None if t is None else t[b:b + 1, :n]
    for b, n in enumerate(lens_l):
        if n >= Lq:
            ref = dsa.indexer_topk(ind["q"][b:b + 1], ind["k"][b:b + 1, :n], ind["w"][b:b + 1], k,
                                   q_scale=sc(ind["q_scale"], b, Lq), k_scale=sc(ind["k_scale"], b, n))
            assert np.array_equal(got[b], ref.cpu().numpy()[0]), (b, n)
        else:   # query i sits at n - Lq + i: only rows with a non-negative position see keys
            for i in range(Lq):
                p = n - Lq + i
                want = list(range(p + 1)) + [-1] * (k - max(p + 1, 0))
                assert got[b, i].tolist() == want[:k], (b, i)
    # the longest sequence against the oracle
    ora = indexer_to_oracle({key: (v[0:1] if torch.is_tensor(v) else v) for key, v in ind.items()})
    rows = [0, Lq - 1]
    osc = _oracle_rows(ora, 0, rows, Lq, Lmax)
    nv = [Lmax - Lq + r + 1 for r in rows]
    ok, _, msg = index_sets_agree(got[0][rows], oracle.topk_rows(osc, nv, k), osc, nv, k, TAU[dtype])
    assert ok, msg


def _to_pool(cache, table, page, pool_pages):
    """Contiguous per-sequence rows [B, Lmax, ...] -> a page pool [pool_pages * page, ...]
    laid out by the block table (unused pool pages hold garbage)."""
    B, max_pages = table.shape
    pool = torch.full((pool_pages * page,) + tuple(cache.shape[2:]), 0x3C if cache.dtype == torch.uint8 else 7,
                      dtype=cache.dtype, device=cache.device)
    for b in range(B):
        for j in range(max_pages):
            pg = int(table[b, j])
            pool[pg * page:(pg + 1) * page] = cache[b, j * page:(j + 1) * page]
    return pool


@pytest.mark.parametrize("dtype,Lq,page", [("fp8", 1, 64), ("bf16", 3, 256)])
def test_paged_decode_equals_contiguous_caches(dtype, Lq, page):
    """Paged k^I / latent caches with a random page permutation (and spare pool pages):
    the index rows equal dsa_indexer_topk_varlen on the contiguous caches, and attention
    over the latent pool through dsa_paged_rows equals attention on the contiguous cache,
    bit for bit."""
    B, Lmax, k = 5, 12800, 512
    cfg = _cfg(dtype, Lmax, k, Lq=Lq, B=B)
    ind = synth.indexer_inputs(cfg, device=DEV)
    lens = torch.tensor([Lmax, 1, 0, 3000, Lmax - 1], dtype=torch.int32, device=DEV)
    max_pages = Lmax // page
    pool_pages = B * max_pages + 7
    rng = np.random.default_rng(21)
    table = torch.from_numpy(rng.permutation(pool_pages)[:B * max_pages].reshape(B, max_pages)
                             .astype(np.int32)).to(DEV)
    kpool = _to_pool(ind["k"], table, page, pool_pages)
    spool = None if ind["k_scale"] is None else _to_pool(ind["k_scale"], table, page, pool_pages)
    idx_v = dsa.indexer_topk_varlen(ind["q"], ind["k"], ind["w"], k, lens, **_ind_args(ind))
    idx_p = dsa.indexer_topk_paged(ind["q"], kpool, ind["w"], k, lens, table, page, q_scale=ind["q_scale"],
                                   k_scale_pool=spool)
    assert torch.equal(idx_p, idx_v)
    rows = dsa.paged_rows(idx_v, table, page, pool_pages)
    iv = idx_v.cpu().numpy()
    tb = table.cpu().numpy()
    want = np.where(iv >= 0, tb[np.arange(B)[:, None, None], np.maximum(iv, 0) // page] * page + iv % page, -1)
    assert np.array_equal(rows.cpu().numpy(), want)
    lay = synth.attention_inputs(cfg, layer=0, device=DEV, Lq=Lq)
    ref = dsa.sparse_attn(lay, idx_v, out_dtype=torch.float32)
    lay_pool = dict(lay)
    lay_pool["q"] = lay["q"].reshape(1, B * Lq, cfg.H, cfg.Dqk)
    lay_pool["kv"] = _to_pool(lay["kv"], table, page, pool_pages)[None]
    got = dsa.sparse_attn(lay_pool, rows.reshape(1, B * Lq, k), out_dtype=torch.float32)
    assert torch.equal(got.reshape(ref.shape), ref)


@pytest.mark.parametrize("dtype,L,k", [("fp8", 12000, 512), ("bf16", 6000, 256)])
def test_future_keys_do_not_change_earlier_rows(dtype, L, k):
    """Causality: overwriting every k^I row, key scale and latent KV row at positions past m
    changes nothing in the index rows and attention outputs of the queries at positions < m
    (bit for bit), through the fused indexer and the MLA kernel at sizes with several work
    items per row and a ragged tail."""
    cfg = _cfg(dtype, L, k)
    ind = synth.indexer_inputs(cfg, device=DEV)
    lay = synth.attention_inputs(cfg, layer=1, device=DEV)
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, **_ind_args(ind))
    out = dsa.sparse_attn(lay, idx, out_dtype=torch.float32)
    m = L // 2 + 37
    ind2 = dict(ind)
    kk = ind["k"].clone()
    if kk.dtype == torch.uint8:
        kk[:, m:] = 0x5A                                  # a finite E4M3 code (72)
    else:
        kk[:, m:] = 3.0
    ind2["k"] = kk
    if ind["k_scale"] is not None:
        ks = ind["k_scale"].clone()
        ks[:, m:] = 7.0
        ind2["k_scale"] = ks
    lay2 = dict(lay)
    kv = lay["kv"].clone()
    kv[:, m:] = -2.0
    lay2["kv"] = kv
    idx2 = dsa.indexer_topk(ind2["q"], ind2["k"], ind2["w"], k, **_ind_args(ind2))
    out2 = dsa.sparse_attn(lay2, idx2, out_dtype=torch.float32)
    assert torch.equal(idx[:, :m], idx2[:, :m])
    assert torch.equal(out[:, :m], out2[:, :m])
    assert not torch.equal(idx[:, m:], idx2[:, m:])       # the later rows did see the change


def test_rows_shorter_than_k_select_every_causal_key():
    cfg = _cfg("fp8", 3000, 2048)
    ind = synth.indexer_inputs(cfg, device=DEV)
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], 2048, **_ind_args(ind)).cpu().numpy()[0]
    for t in (0, 1, 100, 2046, 2047):
        assert idx[t, : t + 1].tolist() == list(range(t + 1))
        assert np.all(idx[t, t + 1:] == -1)
    assert np.all(idx[2048:] >= 0)


# ---------------------------------------------------------------------------
# sparse attention
# ---------------------------------------------------------------------------

def _attn_check(lay, idx_np, out, lse, rows, b=0, idx_rows_override=None):
    ol = attn_to_oracle(lay)
    ir = idx_np[b][rows] if idx_rows_override is None else idx_rows_override
    ref, ref_lse = oracle.sparse_attention_rows(ol["q"][b][rows], ol["k"][b], ol["v"][b], ir,
                                                ol["sm_scale"], ol["Hkv"])
    g = to_f64(out[b][rows])
    rms = math.sqrt(float(np.mean(ref ** 2)))
    err = np.abs(g - ref).max()
    assert err <= 1e-2 * rms, (err, rms)
    if lse is not None:
        gl = lse[b][rows].cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isneginf(gl), np.isneginf(ref_lse))
        fin = np.isfinite(ref_lse)
        assert np.abs(gl[fin] - ref_lse[fin]).max() <= 2e-3 * (1 + np.abs(ref_lse[fin]).max())


def test_mla_prefill_attention_parity():
    L, k = 1500, 256
    cfg = _cfg("bf16", L, k)
    ind = synth.indexer_inputs(cfg, device=DEV)
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, **_ind_args(ind))
    lay = synth.attention_inputs(cfg, layer=1, device=DEV)
    out, lse = dsa.sparse_attn(lay, idx, return_lse=True, out=poisoned((1, L, 32, 512), torch.float32))
    assert all_written(out)
    rows = [0, 1, 5, 255, 256, 700, 1499]
    _attn_check(lay, idx.cpu().numpy(), out, lse, rows)
    out2 = dsa.sparse_attn(lay, idx, out_dtype=torch.float32)
    assert torch.equal(out, out2)                                   # run twice: identical
    out_bf = dsa.sparse_attn(lay, idx)                               # bf16 output = RNE(fp32 result)
    assert out_bf.dtype == torch.bfloat16 and torch.equal(out_bf, out.to(torch.bfloat16))


def test_mla_attention_invalid_and_padded_entries():
    cfg = _cfg("bf16", 300, 40)
    lay = synth.attention_inputs(cfg, layer=0, device=DEV)
    rng = np.random.default_rng(3)
    idx = np.stack([np.sort(rng.permutation(300)[:40]) for _ in range(300)])[None].astype(np.int32)
    idx[0, 0] = -1                         # no key at all: zeros, lse = -inf
    idx[0, 1, 5:] = -1                     # padded row
    idx[0, 2, ::3] = 1000                  # out of range: skipped
    idx[0, 3] = -1
    idx[0, 3, 17] = 7                      # one key: out = V[7]
    out, lse = dsa.sparse_attn(lay, torch.from_numpy(idx).to(DEV), return_lse=True, out_dtype=torch.float32)
    ol_idx = idx.copy()
    ol_idx[ol_idx >= 300] = -1
    rows = [1, 2, 3, 4, 299]
    _attn_check(lay, ol_idx, out, lse, rows)
    assert torch.all(out[0, 0] == 0) and torch.all(torch.isneginf(lse[0, 0]))
    v7 = lay["kv"][0, 7, :512].float()
    assert torch.equal(out[0, 3], v7.expand(32, 512))


def test_mla_decode_split_and_mtp_shared_rows():
    B, Lk, k = 3, 5000, 2048
    cfg = synth.get_config("decode200k", L=Lk, B=B)
    ind = synth.indexer_inputs(cfg, device=DEV)
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, **_ind_args(ind))    # [B, 1, k]
    lay = synth.attention_inputs(cfg, layer=2, device=DEV)                       # Lq = 1
    out, lse = dsa.sparse_attn(lay, idx, return_lse=True, out_dtype=torch.float32)
    for b in range(B):
        _attn_check(lay, idx.cpu().numpy(), out, lse, [0], b=b)
    # MTP draft: 4 queries per sequence share the first step's index row
    lay4 = synth.attention_inputs(cfg, layer=3, device=DEV, Lq=4)
    out4, lse4 = dsa.sparse_attn(lay4, idx, idx_q_stride=0, return_lse=True, out_dtype=torch.float32)
    shared = idx.cpu().numpy()[:, 0]
    for b in range(B):
        _attn_check(lay4, None, out4, lse4, [0, 1, 2, 3], b=b,
                    idx_rows_override=np.repeat(shared[b][None], 4, axis=0))



# The other direction of the attention check: the oracle's own index sets (exact top-k of
# its fp64 scores) fed to dsa_sparse_attn, against the oracle's attention over the same
# sets.  Prefill (bf16 indexer inputs, the two-buffer kernel) and decode (one query per
# sequence, keys split over workgroups).  Rows not checked keep the GPU's index rows.
@pytest.mark.parametrize("case", ["prefill", "decode"])
def test_attention_on_oracle_index_sets(case):
    if case == "prefill":
        L, k, B = 1500, 256, 1
        cfg = _cfg("bf16", L, k)
        rows = [0, 255, 256, 900, 1499]
    else:
        L, k, B = 3000, 2048, 2
        cfg = synth.get_config("decode200k", L=L, B=B)
        rows = [0]
    ind = synth.indexer_inputs(cfg, device=DEV)
    lay = synth.attention_inputs(cfg, layer=2, device=DEV)
    Lq = cfg.Lq
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, **_ind_args(ind)).cpu().numpy()
    ora = indexer_to_oracle(ind)
    ref_idx = {}
    for b in range(B):
        sc = _oracle_rows(ora, b, rows, Lq, L)
        nv = [L - Lq + r + 1 for r in rows]
        ref_idx[b] = oracle.topk_rows(sc, nv, k)
        idx[b][rows] = ref_idx[b]
    out, lse = dsa.sparse_attn(lay, torch.from_numpy(idx).to(DEV), return_lse=True,
                               out=poisoned((B, Lq, cfg.H, cfg.Dv), torch.float32))
    assert all_written(out)
    for b in range(B):
        _attn_check(lay, None, out, lse, rows, b=b, idx_rows_override=ref_idx[b])


def test_decode_step_graph_replays_match_eager():
    """A decode step (fused indexer + top-k, then four layers of sparse attention, one
    workspace) captured as a graph: every kernel is a stream launch (no copies, no memsets,
    no host synchronisation), so each replay, with eager steps in between, reproduces the
    eager step's index rows and outputs bit for bit."""
    cfg = synth.get_config("decode200k", L=20000, B=4)
    k = cfg.topk
    ind = synth.indexer_inputs(cfg, device=DEV)
    layers = [synth.attention_inputs(cfg, layer=l, device=DEV) for l in range(cfg.n_layers)]
    idx = torch.empty((cfg.B, 1, k), dtype=torch.int32, device=DEV)
    outs = [torch.empty((cfg.B, 1, cfg.H, cfg.Dv), dtype=torch.bfloat16, device=DEV) for _ in layers]
    ws = dsa.Workspace()

    def step():
        dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, ws=ws, out=idx, **_ind_args(ind))
        for lay, o in zip(layers, outs):
            dsa.sparse_attn(lay, idx, ws=ws, out=o)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref_idx, ref_outs = idx.clone(), [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        idx.fill_(-7)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx)
        assert all(torch.equal(o, r) for o, r in zip(outs, ref_outs))
        step()                                   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx)

# 48 and 64 query heads take the 16-key kernel (up to eight waves per workgroup): prefill
# rows, decode rows split over several workgroups, and MTP draft queries sharing one row
# (batched per workgroup), against the oracle with the GPU's index rows.
@pytest.mark.parametrize("H", [48, 64])
def test_mla_wide_heads_parity(H):
    rng = np.random.default_rng(H)
    # prefill: 600 queries, 128 keys each from a random causal-looking set
    cfg = synth.get_config("prefill16k", L=600, Lq=600, H=H)
    lay = synth.attention_inputs(cfg, layer=0, device=DEV)
    idx = np.stack([np.sort(rng.permutation(600)[:128]) for _ in range(600)])[None].astype(np.int32)
    idx[0, 3, 100:] = -1
    out, lse = dsa.sparse_attn(lay, torch.from_numpy(idx).to(DEV), return_lse=True,
                               out=poisoned((1, 600, H, 512), torch.float32))
    assert all_written(out)
    _attn_check(lay, idx, out, lse, [0, 3, 299, 599])
    out_bf = dsa.sparse_attn(lay, torch.from_numpy(idx).to(DEV))
    assert torch.equal(out_bf, out.to(torch.bfloat16))
    # decode: 3 sequences x 1 query over 2048 of 5000 keys (keys split over workgroups)
    B, Lk, k = 3, 5000, 2048
    dcfg = synth.get_config("decode200k", L=Lk, B=B, H=H)
    dlay = synth.attention_inputs(dcfg, layer=1, device=DEV)
    didx = np.stack([np.sort(rng.permutation(Lk)[:k]) for _ in range(B)])[:, None].astype(np.int32)
    didx[1, 0, ::9] = -1
    dout, dlse = dsa.sparse_attn(dlay, torch.from_numpy(didx).to(DEV), return_lse=True,
                                 out=poisoned((B, 1, H, 512), torch.float32))
    assert all_written(dout)
    for b in range(B):
        _attn_check(dlay, didx, dout, dlse, [0], b=b)
    # MTP: 4 draft queries per sequence share the row
    mlay = synth.attention_inputs(dcfg, layer=2, device=DEV, Lq=4)
    mout, mlse = dsa.sparse_attn(mlay, torch.from_numpy(didx).to(DEV), idx_q_stride=0, return_lse=True,
                                 out=poisoned((B, 4, H, 512), torch.float32))
    assert all_written(mout)
    for b in range(B):
        _attn_check(mlay, None, mout, mlse, [0, 1, 2, 3], b=b, idx_rows_override=np.repeat(didx[b], 4, axis=0))


# Few query rows take the four-buffer attention (one workgroup per CU, three blocks of 32
# keys in flight, keys split to reach ~256 workgroups).  Cases: splits of one and two
# blocks (fewer than the ring holds), a ragged last block, an unsplit 256-row grid, and
# -1 / out-of-range entries.
@pytest.mark.parametrize("B,Lq,Lk,k,seed", [
    (1, 1, 3000, 2048, 0),      # 8 splits of 8 blocks
    (2, 1, 500, 100, 1),        # 4 blocks, ragged: one block per split
    (2, 1, 900, 520, 2),        # 17 blocks: splits of 3, the last of 2
    (5, 2, 2000, 1000, 3),      # 10 rows, 32 blocks (last ragged), splits of 4
    (4, 1, 2100, 2047, 4),      # ragged 2047
    (1, 256, 400, 300, 5),      # 256 rows: no split, 10 blocks per workgroup
])
def test_mla_deep_ring_edge_cases(B, Lq, Lk, k, seed):
    cfg = synth.get_config("decode200k", L=Lk, B=B)
    lay = synth.attention_inputs(cfg, layer=1, device=DEV, Lq=Lq)
    rng = np.random.default_rng(seed)
    idx = np.stack([np.sort(rng.permutation(Lk)[:k]) for _ in range(B * Lq)]).reshape(B, Lq, k).astype(np.int32)
    idx[0, 0, ::7] = -1                      # holes
    idx[-1, -1, 3::5] = Lk + 11              # out of range: skipped
    if k > 64:
        idx[0, -1, k - 40:] = -1             # padded tail
    out, lse = dsa.sparse_attn(lay, torch.from_numpy(idx).to(DEV), return_lse=True,
                               out=poisoned((B, Lq, 32, 512), torch.float32))
    assert all_written(out)
    ol_idx = idx.copy()
    ol_idx[ol_idx >= Lk] = -1
    for b in range(B):
        rows = sorted({0, Lq - 1, Lq // 2})
        _attn_check(lay, ol_idx, out, lse, rows, b=b)
    out_bf = dsa.sparse_attn(lay, torch.from_numpy(idx).to(DEV))
    assert torch.equal(out_bf, out.to(torch.bfloat16))


# FP8 latent cache: E4M3 codes with one fp32 scale per row (dsa_sparse_attn_kv8), the
# two-buffer (prefill) and four-buffer split (decode) forms, against the oracle on the
# exactly decoded rows
@pytest.mark.parametrize("B,Lq,Lk,k", [(1, 1500, 1500, 256), (3, 1, 5000, 2048), (2, 1, 900, 520)])
def test_mla_fp8_latent_attention_parity(B, Lq, Lk, k):
    cfg = synth.get_config("decode200k", L=Lk, B=B)
    lay = synth.fp8_latent(synth.attention_inputs(cfg, layer=2, device=DEV, Lq=Lq))
    rng = np.random.default_rng(B + k)
    idx = np.stack([np.sort(rng.permutation(min(Lk, Lk - Lq + 1 + i))[:k]) if min(Lk, Lk - Lq + 1 + i) >= k
                    else np.concatenate([np.arange(Lk - Lq + 1 + i), -np.ones(k - (Lk - Lq + 1 + i), np.int64)])
                    for _ in range(B) for i in range(Lq)]).reshape(B, Lq, k).astype(np.int32)
    idx[0, 0, ::11] = -1
    idx[-1, -1, 2::9] = Lk + 5                     # out of range: skipped
    idx_t = torch.from_numpy(idx).to(DEV)
    out, lse = dsa.sparse_attn(lay, idx_t, return_lse=True, out_dtype=torch.float32)
    ol_idx = idx.copy()
    ol_idx[ol_idx >= Lk] = -1
    for b in range(B):
        _attn_check(lay, ol_idx, out, lse, sorted({0, Lq // 2, Lq - 1}), b=b)
    assert torch.equal(out, dsa.sparse_attn(lay, idx_t, out_dtype=torch.float32))     # deterministic
    assert torch.equal(dsa.sparse_attn(lay, idx_t), out.to(torch.bfloat16))


@pytest.mark.parametrize("B,Lq,Lk,k", [(1, 700, 700, 128), (4, 1, 3000, 2048)])
def test_mla_fp8_latent_equals_bf16_on_decoded_rows(B, Lq, Lk, k):
    """With power-of-two row scales the decoded rows are exact in bf16 and every scaling
    in the FP8 path is exact while the probabilities stay normal numbers (codes of at most
    2 and scales 2^-3 .. 2 keep the logits within a few units), so its output equals the
    bf16 path's on the decoded rows bit for bit."""
    cfg = synth.get_config("decode200k", L=Lk, B=B)
    lay = synth.attention_inputs(cfg, layer=3, device=DEV, Lq=Lq)
    rng = np.random.default_rng(7)
    codes = torch.from_numpy((rng.integers(0, 0x41, (B, Lk, 576)) | (rng.integers(0, 2, (B, Lk, 576)) << 7))
                             .astype(np.uint8))
    scale = torch.from_numpy(2.0 ** rng.integers(-3, 2, (B, Lk)).astype(np.float32))
    dec = (codes.view(torch.float8_e4m3fn).float() * scale[..., None]).to(torch.bfloat16)
    lay8 = dict(lay, kv=codes.to(DEV), kv_scale=scale.to(DEV))
    layb = dict(lay, kv=dec.to(DEV))
    idx = torch.from_numpy(np.stack([np.sort(rng.permutation(Lk)[:k]) for _ in range(B * Lq)])
                           .reshape(B, Lq, k).astype(np.int32)).to(DEV)
    got = dsa.sparse_attn(lay8, idx, out_dtype=torch.float32)
    ref = dsa.sparse_attn(layb, idx, out_dtype=torch.float32)
    assert torch.equal(got, ref)



# Draft queries sharing one idx row per sequence (idx_q_stride 0, the MTP case).  With an
# even number per sequence and at most 256 pairs, two queries share a workgroup and the
# rows it gathers (eight waves); an odd number keeps one query per workgroup.  Against the
# oracle on bf16 rows, and on FP8 latent rows bit-exact against the bf16 path on the
# decoded rows (power-of-two scales, as in the test above).
@pytest.mark.parametrize("B,Lq,Lk,k,H", [
    (3, 4, 3000, 2048, 32),     # paired: 6 groups, keys split 8 ways
    (3, 3, 3000, 2048, 32),     # odd count: one query per workgroup
    (127, 2, 700, 300, 32),     # paired: 127 groups, split rounded down to 2
    (2, 4, 900, 520, 16),       # paired, 16 heads: two waves of each query idle
])
def test_mla_shared_row_queries(B, Lq, Lk, k, H):
    cfg = synth.get_config("decode200k", L=Lk, B=B, H=H)
    lay = synth.attention_inputs(cfg, layer=1, device=DEV, Lq=Lq)
    rng = np.random.default_rng(10 * B + Lq)
    idx = np.stack([np.sort(rng.permutation(Lk)[:k]) for _ in range(B)])[:, None].astype(np.int32)
    idx[0, 0, ::13] = -1
    idx[-1, 0, 5::17] = Lk + 3                     # out of range: skipped
    idx_t = torch.from_numpy(idx).to(DEV)
    out, lse = dsa.sparse_attn(lay, idx_t, idx_q_stride=0, return_lse=True,
                               out=poisoned((B, Lq, H, 512), torch.float32))
    assert all_written(out)
    ol_idx = idx.copy()
    ol_idx[ol_idx >= Lk] = -1
    for b in sorted({0, B // 2, B - 1}):
        _attn_check(lay, None, out, lse, list(range(Lq)), b=b, idx_rows_override=np.repeat(ol_idx[b], Lq, axis=0))
    assert torch.equal(dsa.sparse_attn(lay, idx_t, idx_q_stride=0), out.to(torch.bfloat16))
    codes = torch.from_numpy((rng.integers(0, 0x41, (B, Lk, 576)) | (rng.integers(0, 2, (B, Lk, 576)) << 7))
                             .astype(np.uint8))
    scale = torch.from_numpy(2.0 ** rng.integers(-3, 2, (B, Lk)).astype(np.float32))
    dec = (codes.view(torch.float8_e4m3fn).float() * scale[..., None]).to(torch.bfloat16)
    got = dsa.sparse_attn(dict(lay, kv=codes.to(DEV), kv_scale=scale.to(DEV)), idx_t, idx_q_stride=0,
                          out_dtype=torch.float32)
    ref = dsa.sparse_attn(dict(lay, kv=dec.to(DEV)), idx_t, idx_q_stride=0, out_dtype=torch.float32)
    assert torch.equal(got, ref)

def test_tiny_mha_fp32_attention_parity():
    cfg = synth.get_config("tiny")
    ind = synth.indexer_inputs(cfg, device=DEV)
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], cfg.topk, **_ind_args(ind))
    lay = synth.attention_inputs(cfg, layer=0, device=DEV)
    out, lse = dsa.sparse_attn(lay, idx, return_lse=True)
    _attn_check(lay, idx.cpu().numpy(), out, lse, [0, 3, 63, 64, 500, 1023])


# ---------------------------------------------------------------------------
# IndexShare group
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,L,k", [("tiny", 1024, 64), ("prefill16k", 1200, 256), ("prefill128k", 2500, 2048)])
def test_layer_group_shares_full_index_set(name, L, k):
    cfg = synth.get_config(name, L=L, Lq=L, topk=k)
    ind = synth.indexer_inputs(cfg, device=DEV)
    layers = [synth.attention_inputs(cfg, layer=l, device=DEV) for l in range(4)]
    Dv = cfg.Dv
    idx, outs = dsa.layer_group(ind, layers, k, idx_out=poisoned((1, L, k), torch.int32),
                                outs=[poisoned((1, L, cfg.H, Dv), torch.float32) for _ in layers])
    assert all_written(idx) and all(all_written(o) for o in outs)
    idx_alone = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, **_ind_args(ind))
    assert torch.equal(idx, idx_alone)
    for l in range(4):                                                # Shared = standalone on idx_full
        assert torch.equal(outs[l], dsa.sparse_attn(layers[l], idx, out_dtype=torch.float32))
    # oracle on sampled rows: index sets within the band, attention within the bar
    ora = indexer_to_oracle(ind)
    rows = [0, k - 1, min(k, L - 1), L // 2, L - 1]
    sc = _oracle_rows(ora, 0, rows, L, L)
    ref = oracle.topk_rows(sc, [r + 1 for r in rows], k)
    ok, _, msg = index_sets_agree(idx.cpu().numpy()[0][rows], ref, sc, [r + 1 for r in rows], k,
                                  TAU[cfg.idx_dtype])
    assert ok, msg
    for l in (0, 3):
        _attn_check(layers[l], idx.cpu().numpy(), outs[l], None, rows)


# ---------------------------------------------------------------------------
# IndexShare stack: the released schedule (freq 4, offset 3) over 8 layers
# ---------------------------------------------------------------------------

def test_layer_stack_follows_the_schedule():
    L, k, n = 900, 128, 8
    cfg = synth.get_config("prefill16k", L=L, Lq=L, topk=k)
    anchors = dsa.layer_schedule(n, freq=4, offset=3)               # F F F F S S S F
    assert anchors == oracle.anchors(oracle.indexer_types(n, freq=4, offset=3))
    inds = {l: synth.indexer_inputs(cfg, device=DEV, layer=l) for l in range(n) if anchors[l] == l}
    layers = [synth.attention_inputs(cfg, layer=l % 4, device=DEV) for l in range(n)]
    stack = dsa.LayerStack(anchors, k)
    assert stack.n_full == 5
    for l in range(n):
        out = stack.layer(l, layers[l], indexer=inds.get(l), out_dtype=torch.float32)
        a = anchors[l]
        ind = inds[a]
        idx_a = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, **_ind_args(ind))
        assert stack.held == a and torch.equal(stack.idx, idx_a)       # the anchor's set, bitwise
        assert torch.equal(out, dsa.sparse_attn(layers[l], idx_a, out_dtype=torch.float32))
    # a Shared layer whose anchor's set is not held is refused
    fresh = dsa.LayerStack(anchors, k)
    with pytest.raises(RuntimeError):
        fresh.layer(4, layers[4])
    with pytest.raises(ValueError):
        fresh.layer(0, layers[0])
    # oracle on sampled rows of the last Shared layer (anchor 3)
    rows = [0, k - 1, L // 2, L - 1]
    ora = indexer_to_oracle(inds[3])
    sc = _oracle_rows(ora, 0, rows, L, L)
    ref = oracle.topk_rows(sc, [r + 1 for r in rows], k)
    idx3 = dsa.indexer_topk(inds[3]["q"], inds[3]["k"], inds[3]["w"], k, **_ind_args(inds[3]))
    ok, _, msg = index_sets_agree(idx3.cpu().numpy()[0][rows], ref, sc, [r + 1 for r in rows], k, TAU["bf16"])
    assert ok, msg
    out6 = dsa.sparse_attn(layers[6], idx3, out_dtype=torch.float32)
    _attn_check(layers[6], idx3.cpu().numpy(), out6, None, rows)


# ---------------------------------------------------------------------------
# per-token E4M3 quantization (the step before the path): bit-exact
# ---------------------------------------------------------------------------

def _quant_inputs(dtype, T=37, H=64, D=128, seed=8):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, D, generator=g)
    x[3] = 0.0                                    # all-zero token: scale 1, codes 0
    x[5] *= 1e-6                                  # subnormal codes
    x[7] *= 3e4
    x[9, 0, :4] = torch.tensor([-0.0, 1.0, -1.0, 0.0])
    x[11] *= 1e-35                                # scale below 2^-100: quotients by division
    x[13] *= 1e-40                                # subnormal inputs and scale
    return x.to(torch.bfloat16) if dtype == "bf16" else x


# token rows of 8192, 128, 12 and 16384 values
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H,D", [(64, 128), (1, 128), (3, 4), (128, 128)])
def test_quantize_e4m3_bit_exact(dtype, H, D):
    x = _quant_inputs(dtype, H=H, D=D)
    codes, scales = dsa.quantize_e4m3(x.to(DEV))
    ref_c, ref_s = oracle.quantize_e4m3_per_token(x.float().numpy())
    assert np.array_equal(codes.cpu().numpy(), ref_c)
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    # the input generator's route (torch's cast) gives the same bytes
    syn_c, syn_s = synth.encode_e4m3_per_token(x.float())
    assert torch.equal(codes.cpu(), syn_c) and torch.equal(scales.cpu(), syn_s)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("width", [760, 1024])
def test_quantize_e4m3_rounding_boundaries(dtype, width):
    """Quotients on and next to E4M3 rounding boundaries, with scales that are not powers
    of two (amax = 448 * 3 and 448 * 5 / 4): every midpoint between neighbouring codes
    (normal and subnormal), and the neighbouring representable inputs, must round exactly as
    the single-precision quotient does (ties to even).  Rows of 760 values take the
    two-pass kernel, rows of 1024 the register-resident one (reciprocal and correction)."""
    grid = decode_e4m3(np.arange(0x7F, dtype=np.uint8))          # 0 .. 448
    mids = (grid[:-1] + grid[1:]) / 2
    rows = []
    for c in (3.0, 1.25):
        x = np.concatenate([mids * c, -mids * c]).astype(np.float32)
        if dtype == "bf16":
            x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
        near = np.concatenate([np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(-np.inf))])
        row = np.concatenate([[448.0 * c], x, near]).astype(np.float32)
        rows.append(row)
    n = max(len(r) for r in rows)
    assert n <= width
    x = np.zeros((len(rows), width), np.float32)
    for i, r in enumerate(rows):
        x[i, :len(r)] = r
    xt = torch.from_numpy(x)
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
    codes, scales = dsa.quantize_e4m3(xt.to(DEV))
    ref_c, ref_s = oracle.quantize_e4m3_per_token(xt.float().numpy())
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    assert np.array_equal(codes.cpu().numpy(), ref_c)


def test_quantize_appends_to_cache_slot():
    B, Lmax, D, p = 5, 96, 128, 41
    cache = torch.full((B, Lmax, D), 0x5A, dtype=torch.uint8, device=DEV)
    sc_cache = torch.full((B, Lmax), -1.0, dtype=torch.float32, device=DEV)
    new = torch.randn(B, D, device=DEV, dtype=torch.float32)
    dsa.quantize_e4m3(new, codes=cache[:, p], scales=sc_cache[:, p])
    ref_c, ref_s = oracle.quantize_e4m3_per_token(new.cpu().numpy())
    assert np.array_equal(cache[:, p].cpu().numpy(), ref_c)
    assert np.array_equal(sc_cache[:, p].cpu().numpy(), ref_s)
    others = torch.ones(Lmax, dtype=torch.bool)
    others[p] = False
    assert torch.all(cache[:, others] == 0x5A) and torch.all(sc_cache[:, others] == -1.0)


def test_cache_filled_by_quantize_gives_the_indexer_its_operands():
    # prefill writes 700 k^I rows into a 1024-slot cache, three decode steps append one
    # row each; the indexer then reads the cache prefix.  The bytes must equal the input
    # generator's encoding of the same floats, so the selected idx match too.
    cfg = _cfg("fp8", 703, 64)
    Lmax, L0, Lk = 1024, 700, 703
    g = torch.Generator().manual_seed(9)
    kf = torch.randn(Lk, cfg.d_I, generator=g)
    qf = torch.randn(1, cfg.H_I, cfg.d_I, generator=g)
    w = (torch.rand(1, 1, cfg.H_I, generator=g) / cfg.H_I).to(DEV)
    cache = torch.zeros((1, Lmax, cfg.d_I), dtype=torch.uint8, device=DEV)
    sc_cache = torch.zeros((1, Lmax), dtype=torch.float32, device=DEV)
    dsa.quantize_e4m3(kf[:L0].to(DEV), codes=cache[0, :L0], scales=sc_cache[0, :L0])
    for p in range(L0, Lk):
        dsa.quantize_e4m3(kf[p:p + 1].to(DEV), codes=cache[:, p], scales=sc_cache[:, p])
    qc, qs = dsa.quantize_e4m3(qf.to(DEV))
    kc_ref, ks_ref = synth.encode_e4m3_per_token(kf)
    qc_ref, qs_ref = synth.encode_e4m3_per_token(qf)
    assert torch.equal(cache[0, :Lk].cpu(), kc_ref) and torch.equal(sc_cache[0, :Lk].cpu(), ks_ref)
    assert torch.equal(qc.cpu(), qc_ref) and torch.equal(qs.cpu(), qs_ref)
    idx = dsa.indexer_topk(qc.reshape(1, 1, cfg.H_I, cfg.d_I), cache[:, :Lk], w, 64,
                           q_scale=qs.reshape(1, 1), k_scale=sc_cache[:, :Lk])
    idx_ref = dsa.indexer_topk(qc_ref.to(DEV).reshape(1, 1, cfg.H_I, cfg.d_I),
                               kc_ref.to(DEV).reshape(1, Lk, cfg.d_I), w, 64,
                               q_scale=qs_ref.to(DEV).reshape(1, 1),
                               k_scale=ks_ref.to(DEV).reshape(1, Lk))
    assert torch.equal(idx, idx_ref)


# ---------------------------------------------------------------------------
# The step before the path: bf16 linear maps for the indexer's projections
# ---------------------------------------------------------------------------
def _bf16_strided(rows, cols, pad, gen, scale=1.0, ints=False):
    """Seeded bf16 [rows, cols] on the device as a view with row stride cols + pad."""
    if ints:
        full = torch.randint(-8, 9, (rows, cols + pad), generator=gen).float()
    else:
        full = torch.randn(rows, cols + pad, generator=gen) * scale
    return full.to(torch.bfloat16).to(DEV)[:, :cols]


@pytest.mark.parametrize("M,N,K,pad", [(300, 200, 192, 0), (128, 128, 64, 0), (1, 64, 640, 8),
                                       (257, 8192, 256, 16), (4096, 128, 1536, 0)])
def test_linear_bf16_parity(M, N, K, pad):
    """Every output against the oracle's float64 dot product, within the bound of K
    fp32 roundings of the exact products: |y - ref| <= K 2^-24 sum_k |x_k w_k|.  Shapes
    span ragged edges in M and N, one and several K steps, and strided rows."""
    g = torch.Generator().manual_seed(M * 31 + N * 7 + K)
    x = _bf16_strided(M, K, pad, g)
    w = _bf16_strided(N, K, pad, g, scale=0.05)
    y = dsa.linear_bf16(x, w).cpu().numpy().astype(np.float64)
    xo, wo = to_f64(x), to_f64(w)
    ref = oracle.linear(xo, wo)
    bound = K * 2.0 ** -24 * (np.abs(xo) @ np.abs(wo).T) * 1.01 + 1e-30
    err = np.abs(y - ref)
    assert np.all(err <= bound), f"worst excess {np.max(err - bound)}"


def test_linear_bf16_integer_exact():
    """Small-integer operands: every product and partial sum is an integer below 2^24, so
    any fp32 summation order is exact and the result equals the oracle bit for bit."""
    g = torch.Generator().manual_seed(5)
    M, N, K = 200, 136, 512
    x = _bf16_strided(M, K, 0, g, ints=True)
    w = _bf16_strided(N, K, 0, g, ints=True)
    y = dsa.linear_bf16(x, w).cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(y, oracle.linear(to_f64(x), to_f64(w)))


def test_indexer_projections_bit_exact_on_integer_data():
    """The composed projections (three linear maps, then the per-token E4M3 quantization
    of q^I and k^I) equal the oracle's codes, scales and weights exactly when the linear
    maps are exact (integer data), and the operands run through the fused indexer."""
    g = torch.Generator().manual_seed(9)
    T, D, H_I, d_I = 96, 256, 64, 128
    h = _bf16_strided(T, D, 0, g, ints=True)
    wq = _bf16_strided(H_I * d_I, D, 0, g, ints=True)
    wk = _bf16_strided(d_I, D, 0, g, ints=True)
    ww = _bf16_strided(H_I, D, 0, g, ints=True)
    out = dsa.indexer_projections(h, wq, wk, ww, H_I)
    ref = oracle.indexer_projections(to_f64(h), to_f64(wq), to_f64(wk), to_f64(ww), H_I)
    for name in ("q", "k"):
        np.testing.assert_array_equal(out[name].cpu().numpy(), ref[name])
        np.testing.assert_array_equal(out[name + "_scale"].cpu().numpy(), ref[name + "_scale"])
    np.testing.assert_array_equal(out["w"].cpu().numpy().astype(np.float64), ref["w"])
    ind = {"q": out["q"][None], "k": out["k"][None], "w": out["w"][None].contiguous(),
           "q_scale": out["q_scale"][None], "k_scale": out["k_scale"][None]}
    k = 32
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k, q_scale=ind["q_scale"],
                           k_scale=ind["k_scale"]).cpu().numpy()[0]
    ora = indexer_to_oracle(ind)
    rows = list(range(T))
    sc = oracle.indexer_scores_rows(ora["q"][0], ora["k"][0], ora["w"][0], rows, T, ora["q_scale"][0],
                                    ora["k_scale"][0], T)
    ok, _, msg = index_sets_agree(idx, oracle.topk_rows(sc, [r + 1 for r in rows], k), sc, [r + 1 for r in rows], k,
                                  TAU["fp8"])
    assert ok, msg


# ---------------------------------------------------------------------------
# Training of the kept indexer: the group centroid and the KL backward
# ---------------------------------------------------------------------------
def _objective_case(B=2, L=320, k=128, H=32, n_layers=2, H_I=64):
    cfg = synth.get_config("prefill16k", L=L, Lq=L, B=B, topk=k, H=H, H_I=H_I)
    ind = synth.indexer_inputs(cfg, device=DEV)
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k)
    layers = [synth.attention_inputs(cfg, layer=l, device=DEV) for l in range(n_layers)]
    lses = [dsa.sparse_attn(lay, idx, return_lse=True)[1] for lay in layers]
    return cfg, ind, idx, layers, lses


@pytest.mark.parametrize("H", [32, 16])
def test_attention_centroid_parity(H):
    """Each row's centroid of the group's head-averaged distributions on its index row,
    against the oracle's (fp32 exp and MFMA sums of exact bf16 products: relative 1e-4)."""
    cfg, ind, idx, layers, lses = _objective_case(H=H, n_layers=3)
    pbar = dsa.attention_centroid(layers, idx, lses).cpu().numpy()
    idx_h = idx.cpu().numpy()
    for b in range(cfg.B):
        ora_layers = [{"q": attn_to_oracle({**lay, "q": lay["q"][b:b + 1], "kv": lay["kv"][b:b + 1]})["q"][0],
                       "k": attn_to_oracle({**lay, "q": lay["q"][b:b + 1], "kv": lay["kv"][b:b + 1]})["k"][0],
                       "sm_scale": lay["sm_scale"]} for lay in layers]
        ref = oracle.attention_centroid_rows(ora_layers, idx_h[b], list(range(cfg.Lq)))
        np.testing.assert_allclose(pbar[b], ref, rtol=1e-4, atol=1e-7)
        np.testing.assert_allclose(pbar[b].sum(axis=1), 1.0, rtol=1e-4)
        assert np.all(pbar[b][idx_h[b] < 0] == 0)


@pytest.mark.parametrize("H,L,Lq,k,shared", [(32, 300, 300, 100, False), (16, 260, 260, 72, False),
                                              (32, 900, 4, 96, True), (16, 700, 3, 40, True)])
def test_attention_centroid_ragged_and_shared_rows(H, L, Lq, k, shared):
    """The centroid on index rows whose length is not a multiple of the 32-key block, with
    -1 padding on the early rows, and on one index row shared by the queries of a sequence
    (idx_q_stride 0, the MTP-draft case), against the oracle (relative 1e-4)."""
    cfg = synth.get_config("prefill16k", L=L, Lq=Lq, B=2, topk=k, H=H, H_I=64)
    ind = synth.indexer_inputs(cfg, device=DEV)
    idx = dsa.indexer_topk(ind["q"], ind["k"], ind["w"], k)
    if shared:
        idx = idx[:, -1:].contiguous()               # the last query's row, causal for all
    layers = [synth.attention_inputs(cfg, layer=l, device=DEV) for l in range(2)]
    lses = [dsa.sparse_attn(lay, idx, return_lse=True)[1] for lay in layers]
    pbar = dsa.attention_centroid(layers, idx, lses).cpu().numpy()
    idx_h = idx.cpu().numpy()
    for b in range(cfg.B):
        rows_idx = np.repeat(idx_h[b][:1], Lq, axis=0) if shared else idx_h[b]
        ora_layers = [{"q": to_f64(lay["q"][b]), "k": to_f64(lay["kv"][b])[:, None, :], "sm_scale": lay["sm_scale"]}
                      for lay in layers]
        ref = oracle.attention_centroid_rows(ora_layers, rows_idx, list(range(Lq)))
        np.testing.assert_allclose(pbar[b], ref, rtol=1e-4, atol=1e-7)
        assert np.all(pbar[b][rows_idx < 0] == 0)


def test_indexer_kl_backward_dk_is_deterministic():
    """dk sums each key's contributions in 64-bit fixed point, so repeated calls give the
    same bits whatever order the rows arrive in, and a given dk is added to exactly once
    (one fp32 rounding of the sum)."""
    cfg, ind, idx, layers, lses = _objective_case(B=2, L=700, k=256, H_I=64)
    pbar = dsa.attention_centroid(layers, idx, lses)
    runs = [dsa.indexer_kl_backward(ind["q"], ind["k"], ind["w"], idx, pbar) for _ in range(3)]
    for r in runs[1:]:
        for name in ("loss", "dq", "dw", "dk"):
            assert torch.equal(r[name], runs[0][name]), name
    base = torch.randn(ind["k"].shape, device=DEV, dtype=torch.float32)
    added = dsa.indexer_kl_backward(ind["q"], ind["k"], ind["w"], idx, pbar, dk=base.clone())["dk"]
    assert torch.equal(added, base + runs[0]["dk"])


@pytest.mark.parametrize("L,k,H_I", [(320, 128, 64), (200, 100, 32), (150, 64, 16), (130, 50, 48)])
def test_indexer_kl_backward_parity(L, k, H_I):
    """Loss, dq, dw and dk against the oracle on the GPU's centroid.  Bounds: the
    coefficients c = g w [x > 0] enter the contractions rounded to bf16 (relative 2^-9,
    taken as 2^-8 over the sum of |terms|); g = pi - pbar carries the fp32 error of the
    scores and the softmax (1e-4 pi); pre-activations x within the fp32 accumulation error
    of 0 may take either ReLU branch, and their whole term is allowed."""
    cfg, ind, idx, layers, lses = _objective_case(B=2, L=L, k=k, H_I=H_I)
    pbar = dsa.attention_centroid(layers, idx, lses)
    out = dsa.indexer_kl_backward(ind["q"], ind["k"], ind["w"], idx, pbar)
    got = {n: out[n].cpu().numpy().astype(np.float64) for n in out}
    ora = indexer_to_oracle(ind)
    idx_h, pb = idx.cpu().numpy(), pbar.cpu().numpy().astype(np.float64)
    for b in range(cfg.B):
        rows = list(range(cfg.Lq))
        q, kk, w = ora["q"][b], ora["k"][b], ora["w"][b]
        loss, dq, dw, dk = oracle.indexer_kl_rows(q, kk, w, idx_h[b], pb[b], rows)
        bq = np.zeros_like(dq)
        bw = np.zeros_like(dw)
        bk = np.zeros_like(dk)
        for t in rows:
            sel = idx_h[b, t][idx_h[b, t] >= 0]
            x = q[t] @ kk[sel].T
            score = w[t] @ np.maximum(x, 0)
            pi = np.exp(score - score.max()); pi /= pi.sum()
            g = pi - pb[b, t][idx_h[b, t] >= 0]
            dg = 1e-4 * pi + 1e-9
            tau = 2.0 ** -18 * (np.abs(q[t]) @ np.abs(kk[sel]).T)           # x's fp32 error
            near = np.abs(x) <= tau
            c_abs = np.abs(w[t])[:, None] * ((x > 0) | near) * (np.abs(g) + dg)[None, :]
            c_err = 2.0 ** -8 * c_abs + np.abs(w[t])[:, None] * ((x > 0) | near) * dg[None, :] \
                + np.abs(w[t])[:, None] * near * np.abs(g)[None, :]
            bq[t] = c_err @ np.abs(kk[sel])
            np.add.at(bk, sel, c_err.T @ np.abs(q[t]))
            bw[t] = (np.abs(x) * (dg[None, :] + 2.0 ** -16 * np.abs(g)[None, :])).sum(axis=1) \
                + (near * tau * np.abs(g)[None, :]).sum(axis=1)
        np.testing.assert_allclose(got["loss"][b], loss, rtol=1e-4, atol=1e-6)
        for name, g_, r_, bd in (("dq", got["dq"][b], dq, bq), ("dw", got["dw"][b], dw, bw), ("dk", got["dk"][b], dk, bk)):
            err = np.abs(g_ - r_)
            lim = bd + 1e-6 * np.abs(r_).max()
            assert np.all(err <= lim), f"{name}: worst excess {np.max(err - lim)} (max |ref| {np.abs(r_).max()})"
    # the objective is zero with zero gradient when the target is the indexer's own distribution
    own = torch.zeros_like(pbar)
    sc = dsa.indexer_scores(ind["q"], ind["k"], ind["w"])
    for b in range(cfg.B):
        for t in range(cfg.Lq):
            sel = idx[b, t][idx[b, t] >= 0].long()
            own[b, t, : sel.numel()] = torch.softmax(sc[b, t, sel].double(), 0).float()
    z = dsa.indexer_kl_backward(ind["q"], ind["k"], ind["w"], idx, own)
    assert float(z["loss"].abs().max()) < 1e-5
    assert float(z["dw"].abs().max()) < 1e-4 * float(out["dw"].abs().max())
