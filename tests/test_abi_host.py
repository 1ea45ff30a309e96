"""CPU-side checks of the C ABI: the library loads, exports every declared entry point,
sizes workspaces with pure host arithmetic, and rejects invalid arguments before
touching the GPU (these calls return before any HIP call)."""
import ctypes
import os
import re

import pytest

import dsa_lightning_indexer_scores_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

import torch

pytestmark = pytest.mark.skipif(not os.path.exists(dsa.library_path()),
                                reason="libdsa.so not built (run __graft_entry__.build())")

# The error-path tests hand the library fake device addresses and rely on validation
# rejecting the call before any launch; they run only where no GPU is visible.
host_only = pytest.mark.skipif(torch.cuda.device_count() > 0,
                               reason="fake-pointer validation tests run on GPU-less hosts only")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = dsa.load_library()
    names = declared_functions()
    assert set(names) >= {"dsa_indexer_scores", "dsa_topk", "dsa_sparse_attn", "dsa_layer_group",
                          "dsa_indexer_topk", "dsa_workspace_size", "dsa_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in range(0, -7, -1):
        assert dsa.status_string(code).startswith("DSA_")
    assert dsa.status_string(-99) == "unknown dsa_status"


def test_workspace_sizes_are_host_arithmetic():
    ws = dsa.workspace_size
    assert ws(dsa.DSA_OP_TOPK, dsa.DSA_F32, 1, 16, 1000, 64) == 0
    # fp32: one score row per query; decode: one candidate slot (key, position) per key
    assert ws(dsa.DSA_OP_INDEXER_TOPK, dsa.DSA_F32, 1, 1024, 1024, 64) >= 1024 * 1024 * 4
    assert ws(dsa.DSA_OP_INDEXER_TOPK, dsa.DSA_FP8_E4M3, 64, 1, 200001, 2048) >= 64 * 200001 * 8
    # fused: bounded per-workgroup candidate buffers, not Lq x Lk
    big = ws(dsa.DSA_OP_INDEXER_TOPK, dsa.DSA_FP8_E4M3, 1, 131072, 131072, 2048)
    assert 0 < big < 131072 * 131072 * 4 // 16
    # decode attention splits the keys: partial results need a workspace
    assert ws(dsa.DSA_OP_SPARSE_ATTN, dsa.DSA_BF16, 64, 1, 200001, 2048, 32) > 0
    assert ws(dsa.DSA_OP_LAYER_GROUP, dsa.DSA_FP8_E4M3, 64, 1, 200001, 2048, 32) >= \
        ws(dsa.DSA_OP_SPARSE_ATTN, dsa.DSA_BF16, 64, 1, 200001, 2048, 32)
    assert ws(dsa.DSA_OP_INDEXER_TOPK, 7, 1, 16, 16, 4) == 0          # bad dtype
    assert ws(dsa.DSA_OP_INDEXER_TOPK, dsa.DSA_BF16, 1, 32, 16, 4) == 0  # Lq > Lk


def _indexer_struct(dtype=dsa.DSA_BF16, H_I=64, d_I=128, q=0x1000, k=0x2000, w=0x3000, qs=0, ks=0):
    return dsa._IndexerIn(q, qs, k, ks, w, H_I, d_I, dtype)


def _call_indexer_topk(s, B=1, Lq=64, Lk=64, k=16, idx=0x4000, ws=0x10000, nbytes=1 << 40):
    lib = dsa.load_library()
    return lib.dsa_indexer_topk(ctypes.byref(s), B, Lq, Lk, k, idx, ws, nbytes, None)


@host_only
def test_indexer_argument_errors():
    E = {"arg": -1, "dtype": -2, "shape": -3, "align": -4, "ws": -5}
    assert _call_indexer_topk(_indexer_struct(q=0)) == E["arg"]
    assert _call_indexer_topk(_indexer_struct(dtype=9)) == E["dtype"]
    assert _call_indexer_topk(_indexer_struct(H_I=40)) == E["shape"]
    assert _call_indexer_topk(_indexer_struct(d_I=64)) == E["shape"]
    assert _call_indexer_topk(_indexer_struct(q=0x1004)) == E["align"]
    assert _call_indexer_topk(_indexer_struct(dtype=dsa.DSA_FP8_E4M3)) == E["arg"]   # scales missing
    assert _call_indexer_topk(_indexer_struct(), Lq=65, Lk=64) == E["arg"]          # Lq > Lk
    assert _call_indexer_topk(_indexer_struct(), k=0) == E["arg"]
    assert _call_indexer_topk(_indexer_struct(), k=5000) == E["arg"]
    assert _call_indexer_topk(_indexer_struct(), ws=0) == E["ws"]
    assert _call_indexer_topk(_indexer_struct(), nbytes=16) == E["ws"]
    lib = dsa.load_library()
    assert lib.dsa_indexer_scores(ctypes.byref(_indexer_struct()), 1, 4, 4, None, None) == E["arg"]
    assert lib.dsa_topk(None, 8, 1, 8, None, 4, 0x1000, None, None, 0, None) == E["arg"]
    assert lib.dsa_topk(0x1000, 4, 1, 8, None, 4, 0x2000, None, None, 0, None) == E["arg"]  # stride < n
    assert lib.dsa_topk(0x1002, 8, 1, 8, None, 4, 0x2000, None, None, 0, None) == E["align"]


@host_only
def test_indexer_varlen_argument_errors():
    lib = dsa.load_library()
    fp8 = _indexer_struct(dtype=dsa.DSA_FP8_E4M3, qs=0x6000, ks=0x7000)

    def call(s, B=2, Lq=1, Lk=64, lens=0x5000, k=16, idx=0x4000, ws=0x10000, nbytes=1 << 40):
        return lib.dsa_indexer_topk_varlen(ctypes.byref(s), B, Lq, Lk, lens, k, idx, ws, nbytes, None)
    assert call(fp8, lens=0) == -1
    assert call(fp8, idx=0) == -1
    assert call(fp8, k=0) == -1
    assert call(_indexer_struct(dtype=dsa.DSA_F32, H_I=4, d_I=32)) == -2
    assert call(fp8, Lq=16) == -3
    assert call(fp8, lens=0x5002) == -4
    assert call(fp8, ws=0) == -5
    assert call(fp8, nbytes=16) == -5


@host_only
def test_paged_argument_errors():
    lib = dsa.load_library()
    fp8 = _indexer_struct(dtype=dsa.DSA_FP8_E4M3, qs=0x6000, ks=0x7000)

    def call(s, B=2, Lq=1, lens=0x5000, table=0x8000, max_pages=4, page=64, pool=16, k=16, idx=0x4000,
             ws=0x10000, nbytes=1 << 40):
        return lib.dsa_indexer_topk_paged(ctypes.byref(s), B, Lq, lens, table, max_pages, page, pool, k, idx, ws,
                                          nbytes, None)
    assert call(fp8, table=0) == -1
    assert call(fp8, lens=0) == -1
    assert call(fp8, pool=0) == -1
    for bad_page in (32, 96, 100, 1 << 21):
        assert call(fp8, page=bad_page) == -3
    assert call(fp8, Lq=16, max_pages=1) == -3
    assert call(_indexer_struct(dtype=dsa.DSA_F32, H_I=4, d_I=32)) == -2
    assert call(fp8, table=0x8002) == -4
    assert call(fp8, nbytes=16) == -5
    rows = lib.dsa_paged_rows
    assert rows(0, 1, 1, 8, 0x8000, 4, 64, 16, 0x9000, None) == -1
    assert rows(0x4000, 1, 1, 8, 0x8000, 4, 48, 16, 0x9000, None) == -3
    assert rows(0x4002, 1, 1, 8, 0x8000, 4, 64, 16, 0x9000, None) == -4


def _attn_struct(dtype=dsa.DSA_BF16, H=32, Hkv=1, Dqk=576, Dv=512, q=0x1000, k=0x2000, v=0x2000,
                 ks=576, vs=576, out=0x3000):
    return dsa._AttnIn(q, k, ks, v, vs, out, None, H, Hkv, Dqk, Dv, 0.04, dtype)


@host_only
def test_attention_argument_errors():
    lib = dsa.load_library()

    def call(s, idx=0x5000, qstride=16, k=16, ws=0x100000, nbytes=1 << 40, B=1, Lq=4, Lk=64):
        return lib.dsa_sparse_attn(ctypes.byref(s), B, Lq, Lk, idx, qstride, k, ws, nbytes, None)

    assert call(_attn_struct(), idx=0) == -1
    assert call(_attn_struct(), qstride=8) == -1               # 0 < stride < k
    assert call(_attn_struct(H=40)) == -3
    assert call(_attn_struct(Hkv=2)) == -3
    assert call(_attn_struct(Dqk=512)) == -3
    assert call(_attn_struct(v=0x9000)) == -3                   # MLA needs v == k
    assert call(_attn_struct(ks=580, vs=580)) == -4             # stride not multiple of 8
    assert call(_attn_struct(q=0x1008)) == -4
    assert call(_attn_struct(dtype=dsa.DSA_FP8_E4M3)) == -2
    assert call(_attn_struct(dtype=dsa.DSA_F32, H=4, Hkv=4, Dqk=64, Dv=64, ks=256, vs=256), k=9000,
                qstride=9000) == -3
    # decode (few rows) needs the split workspace
    assert call(_attn_struct(), ws=0, nbytes=0, B=2, Lq=1, k=2048, qstride=2048) == -5


@host_only
def test_fp8_latent_attention_argument_errors():
    lib = dsa.load_library()

    def call(s, scale=0x7000, idx=0x5000, ws=0x100000, nbytes=1 << 40, B=1, Lq=4, Lk=64, k=16):
        return lib.dsa_sparse_attn_kv8(ctypes.byref(s), scale, B, Lq, Lk, idx, k, k, ws, nbytes, None)
    assert call(_attn_struct(), scale=0) == -1
    assert call(_attn_struct(), idx=0) == -1
    assert call(_attn_struct(dtype=dsa.DSA_F32, H=4, Hkv=4, Dqk=64, Dv=64, ks=256, vs=256)) == -2
    assert call(_attn_struct(H=48)) == -3                       # 16 or 32 heads only
    assert call(_attn_struct(v=0x9000)) == -3
    assert call(_attn_struct(ks=584, vs=584)) == -4             # code rows: multiple of 16 bytes
    assert call(_attn_struct(), scale=0x7002) == -4
    assert call(_attn_struct(), ws=0, nbytes=0, B=2, Lq=1, k=2048) == -5


@host_only
def test_noalloc_attention_limits():
    # the allocation-free entry point checks its arguments like dsa_sparse_attn and rejects
    # calls whose split partials exceed its device buffer, before any device call
    lib = dsa.load_library()
    limit = 40 << 20

    def call(s, idx=0x5000, B=1, Lq=4, Lk=64, k=16, qstride=16):
        return lib.dsa_sparse_attn_noalloc(ctypes.byref(s), B, Lq, Lk, idx, qstride, k, None)
    assert call(_attn_struct(), idx=0) == -1
    assert call(_attn_struct(H=40)) == -3
    assert call(_attn_struct(q=0x1008)) == -4
    big = dict(B=300, Lq=1, Lk=10 ** 6, k=2048, qstride=2048)    # 300 rows x 32 heads split 4 ways
    assert dsa.workspace_size(dsa.DSA_OP_SPARSE_ATTN, dsa.DSA_BF16, 300, 1, 10 ** 6, 2048, 32) > limit
    assert call(_attn_struct(), **big) == -5
    wide = dict(B=64, Lq=8, Lk=10 ** 5, k=2048, qstride=2048)    # 64 heads, 512 rows split twice
    assert dsa.workspace_size(dsa.DSA_OP_SPARSE_ATTN, dsa.DSA_BF16, 64, 8, 10 ** 5, 2048, 64) > limit
    assert call(_attn_struct(H=64), **wide) == -5


def test_noalloc_buffer_holds_every_decode_shape():
    # every call with at most 32 heads and at most 256 query rows fits the 40 MiB buffer
    worst = max(dsa.workspace_size(dsa.DSA_OP_SPARSE_ATTN, dsa.DSA_BF16, B, Lq, 10 ** 6, k, H)
                for H in (16, 32) for Lq in (1, 2, 4) for B in range(1, 257 // Lq)
                for k in (1, 33, 64, 520, 2047, 2048, 4096))
    assert 0 < worst <= 40 << 20


@host_only
def test_layer_group_argument_errors():
    lib = dsa.load_library()
    full = _indexer_struct()
    layers = (dsa._AttnIn * 2)(_attn_struct(), _attn_struct(H=16))
    st = lib.dsa_layer_group(ctypes.byref(full), layers, 2, 1, 64, 64, 16, 0x4000, 0x100000, 1 << 40, None)
    assert st == -3                                             # layers disagree on H
    st = lib.dsa_layer_group(ctypes.byref(full), None, 1, 1, 64, 64, 16, 0x4000, 0x100000, 1 << 40, None)
    assert st == -1


def test_layer_schedule_matches_the_oracle():
    # host-only entry point: no device memory, callable without a GPU
    import oracle
    for n in (0, 1, 4, 7, 80):
        for freq in (1, 2, 4, 5):
            for off in (0, 1, 3):
                ref = oracle.anchors(oracle.indexer_types(n, freq=freq, offset=off))
                assert dsa.layer_schedule(n, freq=freq, offset=off) == ref, (n, freq, off)
    for pat in ("F", "FSSS", "FFFSSSFS", "FSFSSSSF"):
        assert dsa.layer_schedule(len(pat), pattern=pat) == oracle.anchors(oracle.indexer_types(len(pat), pattern=pat))
    # the released configuration (freq 4, offset 3) over 80 layers: 3 + 20 Full layers
    a = dsa.layer_schedule(80, freq=4, offset=3)
    assert sum(1 for l, x in enumerate(a) if x == l) == 23


@pytest.mark.parametrize("args", [(3, 4, 0, b"SFF"), (3, 4, 0, b"FS"), (3, 4, 0, b"FSSS"), (3, 4, 0, b"FSX"),
                                  (3, 0, 0, None), (3, 4, -1, None), (-1, 4, 0, None)])
def test_layer_schedule_errors(args):
    lib = dsa.load_library()
    out = (ctypes.c_int32 * 8)()
    assert lib.dsa_layer_schedule(*args, out) == -1
    assert lib.dsa_layer_schedule(3, 4, 0, None, None) == -1


@host_only
@pytest.mark.parametrize("args,st", [
    ((0x1000, 5, 4, 128, 128, 0x2000, 128, 0x3000, 1), -2),     # dtype
    ((0x1000, 0, 4, 126, 128, 0x2000, 128, 0x3000, 1), -3),     # row_elems not a multiple of 4
    ((0x1000, 0, 4, 128, 64, 0x2000, 128, 0x3000, 1), -3),      # row stride < row_elems
    ((0x1004, 0, 4, 128, 128, 0x2000, 128, 0x3000, 1), -4),     # fp32 x not 16-byte aligned
    ((0x1000, 0, 4, 128, 128, 0x2001, 128, 0x3000, 1), -4),     # codes not 4-byte aligned
    ((None, 0, 4, 128, 128, 0x2000, 128, 0x3000, 1), -1),
])
def test_quantize_argument_errors(args, st):
    lib = dsa.load_library()
    assert lib.dsa_quantize_e4m3(*args, None) == st


@host_only
@pytest.mark.parametrize("args,st", [
    ((None, 64, 0x2000, 64, 4, 4, 64, 0x3000, 4), -1),          # null x
    ((0x1000, 64, 0x2000, 64, 4, 4, 64, None, 4), -1),          # null y
    ((0x1000, 96, 0x2000, 96, 4, 4, 96, 0x3000, 4), -3),        # K not a multiple of 64
    ((0x1000, 64, 0x2000, 64, 0, 4, 64, 0x3000, 4), -3),        # M = 0
    ((0x1000, 32, 0x2000, 64, 4, 4, 64, 0x3000, 4), -3),        # x row stride < K
    ((0x1000, 64, 0x2000, 64, 4, 8, 64, 0x3000, 4), -3),        # y row stride < N
    ((0x1008, 64, 0x2000, 64, 4, 4, 64, 0x3000, 4), -4),        # x not 16-byte aligned
    ((0x1000, 68, 0x2000, 64, 4, 4, 64, 0x3000, 4), -4),        # x row stride not a multiple of 8
    ((0x1000, 64, 0x2000, 64, 4, 4, 64, 0x3002, 4), -4),        # y not 4-byte aligned
])
def test_linear_argument_errors(args, st):
    lib = dsa.load_library()
    assert lib.dsa_linear_bf16(*args, None) == st


@host_only
def test_objective_argument_errors():
    lib = dsa.load_library()
    s = _attn_struct()
    call = lambda st=s, lse=0x7000, idx=0x5000, P=0x6000, Lk=64, k=16, stride=16: lib.dsa_attn_probs(
        ctypes.byref(st), lse, 1, 4, Lk, idx, stride, k, ctypes.c_float(0.5), P, None)
    assert call(lse=0) == -1
    assert call(P=0) == -1
    assert call(st=_attn_struct(dtype=dsa.DSA_F32, H=4, Hkv=4, Dqk=64, Dv=64, ks=256, vs=256)) == -2
    assert call(st=_attn_struct(H=48)) == -3                    # 16 or 32 heads
    assert call(stride=8) == -3                                 # idx row stride below k
    assert call(P=0x6002) == -4
    ind = _indexer_struct()
    kl = lambda st=ind, k=64, idx=0x5000, dk=0x9000, ws=0x100000, nbytes=1 << 40: lib.dsa_indexer_kl_backward(
        ctypes.byref(st), 1, 8, 64, idx, k, 0x6000, 0x7000, 0x8000, 0x8800, dk, ws, nbytes, None)
    assert kl(idx=0) == -1
    assert kl(dk=0) == -1
    assert kl(st=_indexer_struct(dtype=dsa.DSA_FP8_E4M3, qs=0x100, ks=0x200)) == -2
    assert kl(k=4096) == -3                                     # index rows of at most 2048
    assert kl(st=_indexer_struct(H_I=8)) == -3                  # H_I a multiple of 16
    assert kl(st=_indexer_struct(d_I=64)) == -3                 # d_I = 128
    assert kl(dk=0x9002) == -4
    assert kl(ws=0) == -5
    assert kl(nbytes=64 * 128 * 8 - 1) == -5                   # one int64 per dk element
    assert kl(ws=0x100010) == -4


# ---------------------------------------------------------------------------
# The binding checks dtypes, shapes and batch sizes before a pointer reaches a kernel (a
# kernel indexes every tensor by sizes taken from the others).  The checks run on host
# tensors: a wrong dtype or shape is reported as such, and a correct one gets as far as the
# device check.
# ---------------------------------------------------------------------------

def _raises(fn, *words):
    with pytest.raises(ValueError) as e:
        fn()
    msg = str(e.value)
    assert all(w in msg for w in words), msg


def _fp8_indexer(B=2, Lq=8, Lk=16, H=16, d=128):
    return dict(q=torch.zeros(B, Lq, H, d, dtype=torch.uint8), k=torch.zeros(B, Lk, d, dtype=torch.uint8),
                w=torch.zeros(B, Lq, H), q_scale=torch.ones(B, Lq), k_scale=torch.ones(B, Lk))


def test_binding_checks_indexer_operands():
    good = _fp8_indexer()
    f = lambda **kw: dsa._indexer_struct(**{**good, **kw})
    _raises(lambda: f(), "q", "on the GPU")                                   # passes dtype/shape checks
    _raises(lambda: f(k=torch.zeros(2, 16, 128, dtype=torch.bfloat16)), "k", "dtype")
    _raises(lambda: f(k=torch.zeros(2, 16, 64, dtype=torch.uint8)), "k", "shape")
    _raises(lambda: f(k=torch.zeros(1, 16, 128, dtype=torch.uint8)), "k", "shape")   # batch
    _raises(lambda: f(w=torch.zeros(2, 8, 16, dtype=torch.bfloat16)), "w", "dtype")
    _raises(lambda: f(w=torch.zeros(2, 8, 8)), "w", "shape")
    _raises(lambda: f(q_scale=None), "q_scale", "required")
    _raises(lambda: f(k_scale=torch.ones(2, 15)), "k_scale", "shape")
    _raises(lambda: f(q_scale=torch.ones(2, 8, dtype=torch.float64)), "q_scale", "dtype")
    bf = dict(q=torch.zeros(1, 4, 16, 128, dtype=torch.bfloat16), k=torch.zeros(1, 4, 128, dtype=torch.bfloat16),
              w=torch.zeros(1, 4, 16), q_scale=None, k_scale=None)
    _raises(lambda: dsa._indexer_struct(**bf), "q", "on the GPU")
    _raises(lambda: dsa._indexer_struct(**{**bf, "q_scale": torch.ones(1, 4)}), "scales")
    _raises(lambda: dsa._indexer_struct(**{**bf, "k": torch.zeros(1, 4, 128, dtype=torch.uint8)}), "k", "dtype")


def _mla_layer(B=2, Lq=4, Lk=32, H=32):
    return {"q": torch.zeros(B, Lq, H, 576, dtype=torch.bfloat16), "kv": torch.zeros(B, Lk, 576, dtype=torch.bfloat16),
            "sm_scale": 576 ** -0.5, "Dv": 512}


def test_binding_checks_attention_operands():
    lay = _mla_layer()
    out = torch.zeros(2, 4, 32, 512, dtype=torch.bfloat16)
    _raises(lambda: dsa._attn_struct(lay, out, None), "q", "on the GPU")
    _raises(lambda: dsa._attn_struct({**lay, "kv": torch.zeros(2, 32, 576)}, out, None), "kv", "dtype")
    _raises(lambda: dsa._attn_struct({**lay, "kv": torch.zeros(1, 32, 576, dtype=torch.bfloat16)}, out, None),
            "kv", "shape")
    _raises(lambda: dsa._attn_struct({**lay, "kv": torch.zeros(2, 32, 512, dtype=torch.bfloat16)}, out, None),
            "shorter")
    _raises(lambda: dsa._attn_struct(lay, torch.zeros(2, 4, 32, 512, dtype=torch.float16), None), "out", "dtype")
    _raises(lambda: dsa._attn_struct(lay, torch.zeros(2, 4, 16, 512, dtype=torch.bfloat16), None), "out", "shape")
    _raises(lambda: dsa._attn_struct(lay, out, torch.zeros(2, 4, 16)), "lse", "shape")
    _raises(lambda: dsa._attn_struct(lay, out, torch.zeros(2, 4, 32)), "q", "on the GPU")
    kv8 = {**lay, "kv": torch.zeros(2, 32, 576, dtype=torch.uint8), "kv_scale": torch.ones(2, 31)}
    _raises(lambda: dsa._attn_struct(kv8, out, None), "kv_scale", "shape")
    kv8["kv_scale"] = torch.ones(2, 32)
    _raises(lambda: dsa._attn_struct(kv8, out, None), "q", "on the GPU")
    _raises(lambda: dsa._attn_struct({**kv8, "kv": torch.zeros(2, 32, 576, dtype=torch.bfloat16)}, out, None),
            "kv", "dtype")
    mha = {"q": torch.zeros(1, 4, 4, 64), "k": torch.zeros(1, 8, 2, 64), "v": torch.zeros(1, 8, 2, 32, dtype=torch.bfloat16),
           "sm_scale": 0.125}
    _raises(lambda: dsa._attn_struct(mha, torch.zeros(1, 4, 4, 32), None), "v", "dtype")
    mha["v"] = torch.zeros(1, 8, 2, 32)
    _raises(lambda: dsa._attn_struct(mha, torch.zeros(1, 4, 4, 32), None), "q", "on the GPU")


def test_binding_checks_index_rows():
    _raises(lambda: dsa._check_idx(torch.zeros(2, 4, 64, dtype=torch.int64), 2, 4, 64, 64, None), "idx", "dtype")
    _raises(lambda: dsa._check_idx(torch.zeros(2, 3, 64, dtype=torch.int32), 2, 4, 64, 64, None), "idx", "shape")
    _raises(lambda: dsa._check_idx(torch.zeros(2, 4, 64, dtype=torch.int32), 2, 4, 64, 0, None), "idx", "shape")
    _raises(lambda: dsa._check_idx(torch.zeros(2, 4, 64, dtype=torch.int32), 2, 4, 64, 128, None), "idx_q_stride")
    _raises(lambda: dsa._check_idx(torch.zeros(2, 1, 64, dtype=torch.int32), 2, 4, 64, 0, None), "on the GPU")
    # the public calls check before allocating or launching
    lay = _mla_layer()
    _raises(lambda: dsa.sparse_attn(lay, torch.zeros(2, 4, 64, dtype=torch.int64)), "idx", "dtype")
    _raises(lambda: dsa.topk(torch.zeros(4, 100, dtype=torch.float64), 8), "scores", "dtype")
    _raises(lambda: dsa.topk(torch.zeros(4, 100), 8, n_valid=torch.zeros(4, dtype=torch.int64)), "n_valid", "dtype")
    _raises(lambda: dsa.topk(torch.zeros(4, 100), 8, n_valid=torch.zeros(3, dtype=torch.int32)), "n_valid", "shape")
    ind = _fp8_indexer()
    _raises(lambda: dsa.indexer_topk(ind["q"], ind["k"], ind["w"].double(), 4, q_scale=ind["q_scale"],
                                     k_scale=ind["k_scale"]), "w", "dtype")
    _raises(lambda: dsa.indexer_kl_backward(torch.zeros(1, 4, 16, 128, dtype=torch.bfloat16),
                                            torch.zeros(1, 8, 128, dtype=torch.bfloat16), torch.zeros(1, 4, 16),
                                            torch.zeros(1, 4, 8, dtype=torch.int32), torch.zeros(1, 4, 7)),
            "q", "on the GPU")
