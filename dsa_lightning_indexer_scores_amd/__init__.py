"""Thin Python binding of libdsa.so (DSA lightning indexer -> top-k -> sparse MLA
attention with IndexShare, hand-written HIP kernels for gfx950).

Argument marshalling only: every step of the path runs in the library's kernels.
PyTorch provides device memory and the current stream.  There is no CPU fallback:
if libdsa.so has not been built (``python -m dsa_lightning_indexer_scores_amd.build_lib``)
or no GPU is present, the calls raise.

Function names follow include/dsa.h.
"""
import contextlib
import ctypes
import os

import torch

__all__ = [
    "DSA_F32", "DSA_BF16", "DSA_FP8_E4M3", "DSA_OP_TOPK", "DSA_OP_INDEXER_TOPK",
    "DSA_OP_SPARSE_ATTN", "DSA_OP_LAYER_GROUP", "DSA_OP_INDEXER_KL", "DsaError", "library_path", "load_library",
    "workspace_size", "status_string", "indexer_scores", "topk", "indexer_topk",
    "sparse_attn", "sparse_attn_noalloc", "layer_group", "layer_schedule", "LayerStack", "quantize_e4m3", "linear_bf16", "indexer_projections", "attention_centroid",
    "indexer_kl_backward", "Workspace",
]

DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
DSA_OP_TOPK, DSA_OP_INDEXER_TOPK, DSA_OP_SPARSE_ATTN, DSA_OP_LAYER_GROUP, DSA_OP_INDEXER_KL = 0, 1, 2, 3, 4

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path():
    """libdsa.so next to this file, or the file named by the DSA_LIBRARY variable."""
    return os.environ.get("DSA_LIBRARY") or os.path.join(_HERE, "libdsa.so")


class DsaError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


class _IndexerIn(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("q_scale", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("w", ctypes.c_void_p), ("H_I", ctypes.c_int32),
                ("d_I", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class _AttnIn(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("k_row_stride", ctypes.c_int64),
                ("v", ctypes.c_void_p), ("v_row_stride", ctypes.c_int64), ("out", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("Dqk", ctypes.c_int32), ("Dv", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


_lib = None


def load_library():
    """Load libdsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with "
                           "`python -m dsa_lightning_indexer_scores_amd.build_lib`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.dsa_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.dsa_workspace_size.restype = sz
    lib.dsa_indexer_scores.argtypes = [ctypes.POINTER(_IndexerIn), i32, i32, i32, vp, vp]
    lib.dsa_topk.argtypes = [vp, i64, i32, i32, vp, i32, vp, vp, vp, sz, vp]
    lib.dsa_indexer_topk.argtypes = [ctypes.POINTER(_IndexerIn), i32, i32, i32, i32, vp, vp, sz, vp]
    lib.dsa_indexer_topk_varlen.argtypes = [ctypes.POINTER(_IndexerIn), i32, i32, i32, vp, i32, vp, vp, sz, vp]
    lib.dsa_indexer_topk_paged.argtypes = [ctypes.POINTER(_IndexerIn), i32, i32, vp, vp, i32, i32, i32, i32, vp, vp,
                                           sz, vp]
    lib.dsa_paged_rows.argtypes = [vp, i32, i32, i32, vp, i32, i32, i32, vp, vp]
    lib.dsa_sparse_attn.argtypes = [ctypes.POINTER(_AttnIn), i32, i32, i32, vp, i64, i32, vp, sz, vp]
    lib.dsa_sparse_attn_kv8.argtypes = [ctypes.POINTER(_AttnIn), vp, i32, i32, i32, vp, i64, i32, vp, sz, vp]
    lib.dsa_sparse_attn_noalloc.argtypes = [ctypes.POINTER(_AttnIn), i32, i32, i32, vp, i64, i32, vp]
    lib.dsa_layer_group.argtypes = [ctypes.POINTER(_IndexerIn), ctypes.POINTER(_AttnIn), i32, i32, i32,
                                    i32, i32, vp, vp, sz, vp]
    lib.dsa_layer_schedule.argtypes = [i32, i32, i32, ctypes.c_char_p, ctypes.POINTER(ctypes.c_int32)]
    lib.dsa_quantize_e4m3.argtypes = [vp, i32, i32, i32, i64, vp, i64, vp, i64, vp]
    lib.dsa_linear_bf16.argtypes = [vp, i64, vp, i64, i32, i32, i32, vp, i64, vp]
    lib.dsa_attn_probs.argtypes = [ctypes.POINTER(_AttnIn), vp, i32, i32, i32, vp, i64, i32, ctypes.c_float, vp, vp]
    lib.dsa_indexer_kl_backward.argtypes = [ctypes.POINTER(_IndexerIn), i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp,
                                            sz, vp]
    lib.dsa_status_string.argtypes = [i32]
    lib.dsa_status_string.restype = ctypes.c_char_p
    for fn in ("dsa_indexer_scores", "dsa_topk", "dsa_indexer_topk", "dsa_indexer_topk_varlen",
               "dsa_indexer_topk_paged", "dsa_paged_rows", "dsa_sparse_attn", "dsa_sparse_attn_kv8",
               "dsa_sparse_attn_noalloc", "dsa_layer_group",
               "dsa_layer_schedule", "dsa_quantize_e4m3", "dsa_linear_bf16", "dsa_attn_probs",
               "dsa_indexer_kl_backward"):
        getattr(lib, fn).restype = i32
    _lib = lib
    return lib


def status_string(status):
    return load_library().dsa_status_string(int(status)).decode()


def workspace_size(op, dtype, B, Lq, Lk, k, heads=0):
    return int(load_library().dsa_workspace_size(op, dtype, B, Lq, Lk, k, heads))


def _check(fn, st):
    if st != 0:
        raise DsaError(fn, st)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _alloc_on(stream):
    """Context for the binding's own allocations (outputs, workspace): on the stream the
    kernels will write them, so that torch's caching allocator never hands their memory to
    another stream's tensor while those kernels may still run."""
    if stream is None:
        return contextlib.nullcontext()
    return torch.cuda.stream(stream)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


_FP8_CODES = (torch.uint8, torch.float8_e4m3fn)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype in _FP8_CODES:
        return DSA_FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


def _meta(t, name, dtypes, shape):
    """t must have one of `dtypes` and exactly `shape` (None entries match any size): the
    kernels index every tensor by sizes taken from the others."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if len(t.shape) != len(shape) or any(w is not None and int(g) != int(w) for g, w in zip(t.shape, shape)):
        want = "[" + ", ".join("*" if w is None else str(int(w)) for w in shape) + "]"
        raise ValueError(f"{name} must have shape {want}, not {list(t.shape)}")


def _placed(device, **named):
    """Every given tensor is contiguous and on `device` (checked after dtypes and shapes, so
    those checks also run on host tensors)."""
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous and on the GPU")
        if device is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the call's tensors on {device}")


def _expect(t, name, dtypes, shape, device):
    _meta(t, name, dtypes, shape)
    _placed(device, **{name: t})


class Workspace:
    """A growable device workspace (allocated by torch, handed to the library).  A buffer
    that is replaced may still be read by kernels enqueued on other streams, so each use
    records the stream it is handed to."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes, device, stream=None):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            with _alloc_on(stream):
                self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        if stream is not None:
            self.buf.record_stream(stream)
        return self.buf, self.buf.numel()


def _indexer_struct(q, k, w, q_scale, k_scale, k_batch=None):
    """Checks and packs indexer operands: q [B, Lq, H_I, d_I], k [B', Lk, d_I] of q's dtype
    (B' = k_batch, default B), w float32 [B, Lq, H_I]; for E4M3 codes q_scale float32
    [B, Lq] and k_scale float32 [B', Lk], otherwise no scales."""
    if q is None or q.dim() != 4:
        raise ValueError("q must be [B, Lq, H_I, d_I]")
    dev = q.device
    B, Lq, H_I, d_I = q.shape
    dt = _dtype_code(q)
    kdt = _FP8_CODES if dt == DSA_FP8_E4M3 else (q.dtype,)
    kb = B if k_batch is None else k_batch
    if k is None or k.dim() != 3:
        raise ValueError("k must be [B, Lk, d_I]")
    _meta(k, "k", kdt, (kb, None, d_I))
    Lk = k.shape[1]
    _meta(w, "w", (torch.float32,), (B, Lq, H_I))
    if dt == DSA_FP8_E4M3:
        _meta(q_scale, "q_scale", (torch.float32,), (B, Lq))
        _meta(k_scale, "k_scale", (torch.float32,), (kb, Lk))
    elif q_scale is not None or k_scale is not None:
        raise ValueError("per-token scales belong to E4M3 operands only")
    _placed(dev, q=q, k=k, w=w, q_scale=q_scale, k_scale=k_scale)
    s = _IndexerIn(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w), H_I, d_I, dt)
    return s, B, Lq, Lk


def indexer_scores(q, k, w, q_scale=None, k_scale=None, out=None, stream=None):
    """Materialised scores [B, Lq, Lk] fp32 (-inf for non-causal keys)."""
    s, B, Lq, Lk = _indexer_struct(q, k, w, q_scale, k_scale)
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((B, Lq, Lk), dtype=torch.float32, device=q.device)
    _expect(out, "out", (torch.float32,), (B, Lq, Lk), q.device)
    _check("dsa_indexer_scores", load_library().dsa_indexer_scores(
        ctypes.byref(s), B, Lq, Lk, _ptr(out), _stream(stream)))
    return out


def topk(scores, k, n_valid=None, return_vals=False, ws=None, stream=None):
    """Deterministic top-k over the rows of a 2-D (or batched) fp32 score tensor.  With a
    Workspace, few long rows are split over several workgroups.  n_valid: optional int32
    tensor with one entry per row (the number of leading candidates of that row)."""
    if scores is None or scores.dim() < 1:
        raise ValueError("scores must be a tensor of rows")
    dev = scores.device
    _meta(scores, "scores", (torch.float32,), tuple(scores.shape))
    n = scores.shape[-1]
    rows = scores.numel() // n if n else 0
    if n_valid is not None:
        _meta(n_valid, "n_valid", (torch.int32,), tuple(scores.shape[:-1]))
    _placed(dev, scores=scores, n_valid=n_valid)
    with _alloc_on(stream):
        idx = torch.empty(scores.shape[:-1] + (k,), dtype=torch.int32, device=dev)
        vals = torch.empty(idx.shape, dtype=torch.float32, device=dev) if return_vals else None
    buf, nbytes = None, 0
    if ws is not None:
        buf, nbytes = ws.get(workspace_size(DSA_OP_TOPK, 0, 1, rows, n, k), dev, stream)
    _check("dsa_topk", load_library().dsa_topk(
        _ptr(scores), n, rows, n, _ptr(n_valid), k, _ptr(idx), _ptr(vals), _ptr(buf), nbytes, _stream(stream)))
    return (idx, vals) if return_vals else idx


def _idx_out(out, B, Lq, topk_k, device, stream):
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((B, Lq, topk_k), dtype=torch.int32, device=device)
    _expect(out, "out", (torch.int32,), (B, Lq, topk_k), device)
    return out


def indexer_topk(q, k, w, topk_k, q_scale=None, k_scale=None, ws=None, out=None, stream=None):
    """Fused indexer + top-k: idx [B, Lq, topk_k] int32."""
    s, B, Lq, Lk = _indexer_struct(q, k, w, q_scale, k_scale)
    need = workspace_size(DSA_OP_INDEXER_TOPK, s.dtype, B, Lq, Lk, topk_k)
    ws = ws or Workspace()
    buf, nbytes = ws.get(need, q.device, stream)
    out = _idx_out(out, B, Lq, topk_k, q.device, stream)
    _check("dsa_indexer_topk", load_library().dsa_indexer_topk(
        ctypes.byref(s), B, Lq, Lk, topk_k, _ptr(out), _ptr(buf), nbytes, _stream(stream)))
    return out


def indexer_topk_varlen(q, k, w, topk_k, seq_lens, q_scale=None, k_scale=None, ws=None, out=None, stream=None):
    """Decode indexer + top-k over caches of different lengths: k [B, Lk_max, d_I] of which
    sequence b holds the first seq_lens[b] rows (seq_lens: int32 [B] on the device).
    idx [B, Lq, topk_k] int32; Lq < 16."""
    s, B, Lq, Lk = _indexer_struct(q, k, w, q_scale, k_scale)
    _expect(seq_lens, "seq_lens", (torch.int32,), (B,), q.device)
    need = workspace_size(DSA_OP_INDEXER_TOPK, s.dtype, B, Lq, Lk, topk_k)
    ws = ws or Workspace()
    buf, nbytes = ws.get(need, q.device, stream)
    out = _idx_out(out, B, Lq, topk_k, q.device, stream)
    _check("dsa_indexer_topk_varlen", load_library().dsa_indexer_topk_varlen(
        ctypes.byref(s), B, Lq, Lk, _ptr(seq_lens), topk_k, _ptr(out), _ptr(buf), nbytes, _stream(stream)))
    return out


def indexer_topk_paged(q, k_pool, w, topk_k, seq_lens, block_table, page_size, q_scale=None, k_scale_pool=None,
                       ws=None, out=None, stream=None):
    """Decode indexer + top-k over paged caches: k_pool [pool_pages * page_size, d_I] (and
    k_scale_pool [pool_pages * page_size] for fp8), block_table int32 [B, max_pages] of
    page ids, seq_lens int32 [B].  Returns positions idx [B, Lq, topk_k] int32; Lq < 16."""
    if q is None or q.dim() != 4:
        raise ValueError("q must be [B, Lq, H_I, d_I]")
    B = q.shape[0]
    if k_pool is None or k_pool.dim() != 2 or page_size <= 0 or k_pool.shape[0] % page_size:
        raise ValueError("k_pool must be [pool_pages * page_size, d_I]")
    if block_table is None or block_table.dim() != 2:
        raise ValueError("block_table must be a contiguous int32 [B, max_pages]")
    _expect(block_table, "block_table", (torch.int32,), (B, None), q.device)
    _expect(seq_lens, "seq_lens", (torch.int32,), (B,), q.device)
    max_pages, pool_pages = block_table.shape[1], k_pool.shape[0] // page_size
    s, _, Lq, _ = _indexer_struct(q, k_pool[None], w, q_scale,
                                  None if k_scale_pool is None else k_scale_pool[None], k_batch=1)
    need = workspace_size(DSA_OP_INDEXER_TOPK, s.dtype, B, Lq, max_pages * page_size, topk_k)
    ws = ws or Workspace()
    buf, nbytes = ws.get(need, q.device, stream)
    out = _idx_out(out, B, Lq, topk_k, q.device, stream)
    _check("dsa_indexer_topk_paged", load_library().dsa_indexer_topk_paged(
        ctypes.byref(s), B, Lq, _ptr(seq_lens), _ptr(block_table), max_pages, page_size, pool_pages, topk_k,
        _ptr(out), _ptr(buf), nbytes, _stream(stream)))
    return out


def paged_rows(idx, block_table, page_size, pool_pages, out=None, stream=None):
    """Positions idx [B, Lq, k] -> pool rows [B, Lq, k] (dsa_paged_rows), for dsa_sparse_attn
    over a latent page pool (call it with the queries as one batch of B * Lq)."""
    if idx is None or idx.dim() != 3:
        raise ValueError("idx must be int32 [B, Lq, k]")
    _expect(idx, "idx", (torch.int32,), tuple(idx.shape), idx.device)
    B, Lq, k = idx.shape
    if block_table is None or block_table.dim() != 2:
        raise ValueError("block_table must be a contiguous int32 [B, max_pages]")
    _expect(block_table, "block_table", (torch.int32,), (B, None), idx.device)
    if out is None:
        with _alloc_on(stream):
            out = torch.empty_like(idx)
    _expect(out, "out", (torch.int32,), (B, Lq, k), idx.device)
    _check("dsa_paged_rows", load_library().dsa_paged_rows(
        _ptr(idx), B, Lq, k, _ptr(block_table), block_table.shape[1], page_size, pool_pages, _ptr(out),
        _stream(stream)))
    return out


def _attn_struct(layer, out, lse):
    """Checks and packs one layer's attention operands: q [B, Lq, H, Dqk]; an MLA latent
    cache kv [B, Lk, row] (q's dtype, or uint8 E4M3 codes with kv_scale float32 [B, Lk]),
    or k [B, Lk, Hkv, Dqk] and v [B, Lk, Hkv, Dv] of q's dtype; out [B, Lq, H, Dv] float32 or
    q's dtype; lse float32 [B, Lq, H] or None.  Returns (struct, Lk, Dv)."""
    q = layer.get("q")
    if q is None or q.dim() != 4:
        raise ValueError("q must be [B, Lq, H, Dqk]")
    dev = q.device
    B, Lq, H, Dqk = q.shape
    _meta(q, "q", (torch.bfloat16, torch.float32), (B, Lq, H, Dqk))
    sc = None
    if "kv" in layer:                        # MLA latent: k = v = kv rows, V = first Dv dims
        kk = vv = layer["kv"]
        if kk is None or kk.dim() != 3:
            raise ValueError("kv must be [B, Lk, row]")
        sc = layer.get("kv_scale")
        _meta(kk, "kv", (torch.uint8,) if sc is not None else (q.dtype,), (B, None, None))
        Hkv = 1
        Dv = layer.get("Dv", 512)
        ks = vs = kk.shape[-1]
        if ks < Dqk:
            raise ValueError(f"latent rows of {ks} values are shorter than the query's {Dqk}")
        if sc is not None:
            _meta(sc, "kv_scale", (torch.float32,), (B, kk.shape[1]))
    else:
        kk, vv = layer.get("k"), layer.get("v")
        if kk is None or vv is None or kk.dim() != 4 or vv.dim() != 4:
            raise ValueError("k must be [B, Lk, Hkv, Dqk] and v [B, Lk, Hkv, Dv]")
        Hkv, Dv = kk.shape[2], vv.shape[-1]
        _meta(kk, "k", (q.dtype,), (B, None, Hkv, Dqk))
        _meta(vv, "v", (q.dtype,), (B, kk.shape[1], Hkv, Dv))
        ks, vs = Hkv * Dqk, Hkv * Dv
    _meta(out, "out", (torch.float32, q.dtype), (B, Lq, H, Dv))
    if lse is not None:
        _meta(lse, "lse", (torch.float32,), (B, Lq, H))
    _placed(dev, q=q, k=kk, v=vv, kv_scale=sc, out=out, lse=lse)
    return _AttnIn(_ptr(q), _ptr(kk), ks, _ptr(vv), vs, _ptr(out), _ptr(lse), H, Hkv, Dqk, Dv,
                   float(layer["sm_scale"]), _dtype_code(q), _dtype_code(out)), kk.shape[1], Dv


def _check_idx(idx, B, Lq, k, idx_q_stride, device):
    """idx int32 [B, Lq, k] read with idx_q_stride = k, or [B, 1, k] shared by the Lq queries
    (idx_q_stride = 0, the MTP-draft reuse)."""
    if idx is None or idx.dim() != 3:
        raise ValueError("idx must be int32 [B, Lq, k] or [B, 1, k]")
    if idx_q_stride == 0:
        _meta(idx, "idx", (torch.int32,), (B, 1, k))
    elif idx_q_stride == k:
        _meta(idx, "idx", (torch.int32,), (B, Lq, k))
    else:
        raise ValueError(f"idx_q_stride must be 0 or k = {k} for a contiguous idx")
    _placed(device, idx=idx)


def sparse_attn(layer, idx, idx_q_stride=None, return_lse=False, ws=None, out=None, out_dtype=None,
                stream=None):
    """Sparse attention of one layer over the positions in idx.

    layer: dict with q [B,Lq,H,Dqk], sm_scale, and either kv [B,Lk,576] (MLA latent, V = first
    512 dims; uint8 E4M3 codes with kv_scale [B,Lk] float32 for an FP8 latent cache) or
    k [B,Lk,Hkv,Dqk] and v [B,Lk,Hkv,Dv].  idx: [B,Lq,k] int32, or [B,1,k] with
    idx_q_stride=0 (all queries share the row, the MTP-draft case).  out_dtype: torch.float32
    keeps the fp32 result; default is q's dtype.
    """
    q = layer["q"]
    if q is None or q.dim() != 4 or idx is None or idx.dim() != 3:
        raise ValueError("q must be [B, Lq, H, Dqk] and idx [B, Lq | 1, k]")
    B, Lq, H = q.shape[0], q.shape[1], q.shape[2]
    k = idx.shape[-1]
    if idx_q_stride is None:
        idx_q_stride = 0 if idx.shape[1] == 1 and Lq > 1 else k
    _check_idx(idx, B, Lq, k, idx_q_stride, q.device)
    Dv = layer.get("Dv", 512) if "kv" in layer else layer["v"].shape[-1]
    with _alloc_on(stream):
        if out is None:
            out = torch.empty((B, Lq, H, Dv), dtype=out_dtype or q.dtype, device=q.device)
        lse = torch.empty((B, Lq, H), dtype=torch.float32, device=q.device) if return_lse else None
    s, Lk, _ = _attn_struct(layer, out, lse)
    need = workspace_size(DSA_OP_SPARSE_ATTN, s.dtype, B, Lq, Lk, k, H)
    ws = ws or Workspace()
    buf, nbytes = ws.get(need, q.device, stream)
    if layer.get("kv_scale") is not None:
        _check("dsa_sparse_attn_kv8", load_library().dsa_sparse_attn_kv8(
            ctypes.byref(s), _ptr(layer["kv_scale"]), B, Lq, Lk, _ptr(idx), idx_q_stride, k, _ptr(buf), nbytes,
            _stream(stream)))
    else:
        _check("dsa_sparse_attn", load_library().dsa_sparse_attn(
            ctypes.byref(s), B, Lq, Lk, _ptr(idx), idx_q_stride, k, _ptr(buf), nbytes, _stream(stream)))
    return (out, lse) if return_lse else out


def sparse_attn_noalloc(layer, idx, out, lse=None, idx_q_stride=None, stream=None):
    """sparse_attn through dsa_sparse_attn_noalloc: the split-key partials go to the library's
    own device buffer, so the call allocates nothing.  out [B, Lq, H, Dv] (and lse
    [B, Lq, H] float32, optional) are the caller's; bf16 latent caches only.  Calls that
    overlap on one GPU race (they share the buffer)."""
    q = layer["q"]
    if q is None or q.dim() != 4 or idx is None or idx.dim() != 3:
        raise ValueError("q must be [B, Lq, H, Dqk] and idx [B, Lq | 1, k]")
    if layer.get("kv_scale") is not None:
        raise ValueError("dsa_sparse_attn_noalloc takes bf16 latent caches")
    B, Lq = q.shape[0], q.shape[1]
    k = idx.shape[-1]
    if idx_q_stride is None:
        idx_q_stride = 0 if idx.shape[1] == 1 and Lq > 1 else k
    _check_idx(idx, B, Lq, k, idx_q_stride, q.device)
    s, Lk, _ = _attn_struct(layer, out, lse)
    _check("dsa_sparse_attn_noalloc", load_library().dsa_sparse_attn_noalloc(
        ctypes.byref(s), B, Lq, Lk, _ptr(idx), idx_q_stride, k, _stream(stream)))
    return out


def layer_group(full, layers, topk_k, ws=None, return_lse=False, outs=None, idx_out=None, out_dtype=None,
                stream=None):
    """One IndexShare group: the Full layer's indexer + top-k once, then every layer's
    sparse attention with that index set.  full: dict(q, k, w, q_scale, k_scale);
    layers: list of attention dicts as for sparse_attn.  Returns (idx, [out per layer])."""
    s, B, Lq, Lk = _indexer_struct(full["q"], full["k"], full["w"], full.get("q_scale"), full.get("k_scale"))
    dev = full["q"].device
    n = len(layers)
    structs = (_AttnIn * max(n, 1))()
    with _alloc_on(stream):
        if outs is None:
            outs = []
            for lay in layers:
                q = lay["q"]
                Dv = lay.get("Dv", 512) if "kv" in lay else lay["v"].shape[-1]
                outs.append(torch.empty((q.shape[0], q.shape[1], q.shape[2], Dv), dtype=out_dtype or q.dtype,
                                        device=q.device))
        lses = [torch.empty(lay["q"].shape[:3], dtype=torch.float32, device=lay["q"].device) if return_lse
                else None for lay in layers]
    if len(outs) != n:
        raise ValueError("one output per layer is required")
    for i, lay in enumerate(layers):
        if lay.get("kv_scale") is not None:
            raise ValueError("dsa_layer_group takes bf16 latent caches (FP8 latent layers run through sparse_attn)")
        st, Lk_l, _ = _attn_struct(lay, outs[i], lses[i])
        if lay["q"].shape[:2] != (B, Lq) or Lk_l != Lk:
            raise ValueError(f"layer {i}: its q and cache must cover the indexer's B, Lq and Lk")
        structs[i] = st
    idx_out = _idx_out(idx_out, B, Lq, topk_k, dev, stream)
    heads = layers[0]["q"].shape[2] if n else 16
    need = workspace_size(DSA_OP_LAYER_GROUP, s.dtype, B, Lq, Lk, topk_k, heads)
    ws = ws or Workspace()
    buf, nbytes = ws.get(need, dev, stream)
    _check("dsa_layer_group", load_library().dsa_layer_group(
        ctypes.byref(s), structs, n, B, Lq, Lk, topk_k, _ptr(idx_out), _ptr(buf), nbytes, _stream(stream)))
    if return_lse:
        return idx_out, outs, lses
    return idx_out, outs


def layer_schedule(n_layers, freq=4, offset=0, pattern=None):
    """Anchor of every layer of an IndexShare stack (dsa_layer_schedule): the Full layer
    whose index set the layer attends with; a layer is Full when it is its own anchor.
    pattern: optional string of 'F' / 'S', one per layer (then freq and offset are unused)."""
    out = (ctypes.c_int32 * max(int(n_layers), 1))()
    st = load_library().dsa_layer_schedule(int(n_layers), int(freq), int(offset),
                                           None if pattern is None else pattern.encode(), out)
    if st < 0:
        raise DsaError("dsa_layer_schedule", st)
    return [int(a) for a in out[:n_layers]]


class LayerStack:
    """The layers of an IndexShare stack, run one call per layer in layer order (the way a
    model's forward pass reaches them).  A Full layer runs the indexer + top-k on its own
    operands into the stack's index buffer and then its sparse attention; a Shared layer
    runs only its sparse attention, with the set its anchor left in the buffer.

    anchors: as returned by layer_schedule.  topk_k: k of the top-k.
    """

    def __init__(self, anchors, topk_k, ws=None):
        self.anchors = list(anchors)
        self.k = int(topk_k)
        self.ws = ws or Workspace()
        self.idx = None
        self.held = None          # the Full layer whose set is in self.idx

    def is_full(self, layer):
        return self.anchors[layer] == layer

    @property
    def n_full(self):
        return sum(1 for l in range(len(self.anchors)) if self.is_full(l))

    def layer(self, l, attn, indexer=None, out=None, out_dtype=None, stream=None):
        """Run layer l.  attn: the layer's attention operands (as for sparse_attn);
        indexer: its indexer operands (dict q, k, w, q_scale, k_scale), required for a Full
        layer and ignored for a Shared one.  Returns the attention output."""
        if self.is_full(l):
            if indexer is None:
                raise ValueError(f"layer {l} is a Full layer: its indexer operands are required")
            q = indexer["q"]
            shape = (q.shape[0], q.shape[1], self.k)
            if self.idx is None or tuple(self.idx.shape) != shape or self.idx.device != q.device:
                with _alloc_on(stream):
                    self.idx = torch.empty(shape, dtype=torch.int32, device=q.device)
            indexer_topk(q, indexer["k"], indexer["w"], self.k, q_scale=indexer.get("q_scale"),
                         k_scale=indexer.get("k_scale"), ws=self.ws, out=self.idx, stream=stream)
            self.held = l
        elif self.held != self.anchors[l]:
            raise RuntimeError(f"layer {l} attends with the set of layer {self.anchors[l]}, "
                               f"but the stack holds the set of layer {self.held}")
        return sparse_attn(attn, self.idx, ws=self.ws, out=out, out_dtype=out_dtype, stream=stream)


def quantize_e4m3(x, codes=None, scales=None, stream=None):
    """Per-token E4M3 quantization (dsa_quantize_e4m3): x [T, ...] float32 or bfloat16,
    one token per leading index.  Returns (codes uint8 [T, ...], scales float32 [T]).
    codes / scales may be given as 2-D [T, n] / 1-D [T] views with a row stride (e.g. the
    slot of a decode step in a k^I cache: cache[:, p] and scale_cache[:, p])."""
    _require_cuda(x)
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    T = x.shape[0]
    n = x[0].numel() if T > 0 else 0
    x2 = x.reshape(T, n)
    if x2.stride(1) != 1:
        raise ValueError("each token's values must be contiguous")
    if codes is None:
        with _alloc_on(stream):
            codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    c2 = codes.view(T, n) if codes.dim() != 2 else codes     # view: never a silent copy
    if c2.dtype != torch.uint8 or tuple(c2.shape) != (T, n) or c2.stride(1) != 1:
        raise ValueError("codes must be uint8 [T, n] with contiguous rows")
    if scales is None:
        with _alloc_on(stream):
            scales = torch.empty(T, dtype=torch.float32, device=x.device)
    if not (codes.is_cuda and scales.is_cuda) or codes.device != x.device or scales.device != x.device:
        raise ValueError("codes and scales must be on x's GPU")
    if scales.dtype != torch.float32 or tuple(scales.shape) != (T,):
        raise ValueError("scales must be float32 [T]")
    _check("dsa_quantize_e4m3", load_library().dsa_quantize_e4m3(
        _ptr(x2), DSA_BF16 if x.dtype == torch.bfloat16 else DSA_F32, T, n, x2.stride(0), _ptr(c2), c2.stride(0),
        _ptr(scales), scales.stride(0), _stream(stream)))
    return codes, scales


def linear_bf16(x, w, out=None, stream=None):
    """y = x w^T (dsa_linear_bf16): x bfloat16 [M, K] with contiguous rows, w bfloat16
    [N, K] (a linear layer's weight), K a multiple of 64; returns float32 [M, N].  Rows may
    be strided (views of wider tensors) but their elements must be contiguous."""
    if not (x.is_cuda and w.is_cuda):
        raise ValueError("x and w must be on the GPU")
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("x and w must be bfloat16")
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1] or x.stride(1) != 1 or w.stride(1) != 1:
        raise ValueError("x [M, K] and w [N, K] with contiguous rows are required")
    M, K = x.shape
    N = w.shape[0]
    if x.device != w.device:
        raise ValueError("x and w must be on the same GPU")
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if not out.is_cuda or out.device != x.device or out.dtype != torch.float32 or tuple(out.shape) != (M, N) or out.stride(1) != 1:
        raise ValueError("out must be float32 [M, N] with contiguous rows")
    _check("dsa_linear_bf16", load_library().dsa_linear_bf16(
        _ptr(x), x.stride(0), _ptr(w), w.stride(0), M, N, K, _ptr(out), out.stride(0), _stream(stream)))
    return out


def indexer_projections(h, wq, wk, ww, H_I, stream=None):
    """The indexer's operands from hidden states h bfloat16 [T, D]: q^I = h wq^T
    (wq [H_I * d_I, D]) and k^I = h wk^T (wk [d_I, D]) in fp32, each quantized per token to
    E4M3 (dsa_quantize_e4m3), and the head weights w = h ww^T (ww [H_I, D]) in fp32.
    Returns dict(q [T, H_I, d_I] uint8, q_scale [T], k [T, d_I] uint8, k_scale [T],
    w [T, H_I] float32) -- the per-sequence operands of indexer_topk after a [None]."""
    T = h.shape[0]
    d_I = wk.shape[0]
    if wq.shape[0] != H_I * d_I or ww.shape[0] != H_I:
        raise ValueError("wq must be [H_I * d_I, D] and ww [H_I, D]")
    q32 = linear_bf16(h, wq, stream=stream)
    k32 = linear_bf16(h, wk, stream=stream)
    w32 = linear_bf16(h, ww, stream=stream)
    q, q_scale = quantize_e4m3(q32.view(T, H_I, d_I), stream=stream)
    k, k_scale = quantize_e4m3(k32, stream=stream)
    return {"q": q, "q_scale": q_scale, "k": k, "k_scale": k_scale, "w": w32}


def attention_centroid(layers, idx, lses, idx_q_stride=None, out=None, stream=None):
    """The centroid of the group's attention distributions on each query's index row
    (dsa_attn_probs once per layer, weight 1/len(layers)): each layer's distribution is the
    mean over its heads of the softmax over the row, rebuilt from the layer's q, latent kv,
    sm_scale and the lse its sparse_attn returned for the same idx.  layers: MLA layer
    dicts (bf16 q [B,Lq,H,576], kv [B,Lk,576]); lses: one [B,Lq,H] float32 per layer.
    Returns pbar float32 [B, Lq, k] (0 at -1 entries)."""
    if len(layers) == 0 or len(lses) != len(layers):
        raise ValueError("one lse per layer is required")
    q0 = layers[0]["q"]
    if q0 is None or q0.dim() != 4 or idx is None or idx.dim() != 3:
        raise ValueError("q must be [B, Lq, H, 576] and idx [B, Lq | 1, k]")
    dev = q0.device
    B, Lq = q0.shape[0], q0.shape[1]
    k = idx.shape[-1]
    if idx_q_stride is None:
        idx_q_stride = 0 if idx.shape[1] == 1 and Lq > 1 else k
    _check_idx(idx, B, Lq, k, idx_q_stride, dev)
    if out is None:
        with _alloc_on(stream):
            out = torch.zeros((B, Lq, k), dtype=torch.float32, device=dev)
    _expect(out, "out", (torch.float32,), (B, Lq, k), dev)
    alpha = 1.0 / len(layers)
    for lay, lse in zip(layers, lses):
        q, kv = lay["q"], lay.get("kv")
        if q is None or q.dim() != 4 or kv is None or kv.dim() != 3:
            raise ValueError("each layer needs q [B, Lq, H, 576] and a latent kv [B, Lk, row]")
        H = q.shape[2]
        _expect(q, "q", (torch.bfloat16,), (B, Lq, H, q.shape[3]), dev)
        _expect(kv, "kv", (torch.bfloat16,), (B, None, None), dev)
        _expect(lse, "lse", (torch.float32,), (B, Lq, H), dev)
        s = _AttnIn(_ptr(q), _ptr(kv), kv.shape[-1], _ptr(kv), kv.shape[-1], None, _ptr(lse), H, 1,
                    q.shape[-1], lay.get("Dv", 512), float(lay["sm_scale"]), _dtype_code(q), _dtype_code(q))
        _check("dsa_attn_probs", load_library().dsa_attn_probs(
            ctypes.byref(s), _ptr(lse), B, Lq, kv.shape[1], _ptr(idx), idx_q_stride, k, alpha, _ptr(out),
            _stream(stream)))
    return out


def indexer_kl_backward(q, k, w, idx, pbar, dk=None, ws=None, stream=None):
    """Loss and gradients of the group-centroid objective of the kept indexer
    (dsa_indexer_kl_backward): q bf16 [B,Lq,H_I,128], k bf16 [B,Lk,128], w float32
    [B,Lq,H_I], idx int32 [B,Lq,k], pbar float32 [B,Lq,k].  Returns dict(loss [B,Lq],
    dq [B,Lq,H_I,128], dw [B,Lq,H_I], dk [B,Lk,128]); dk, if given, is added to.  dk does
    not depend on the order of the rows' additions (fixed-point sums in the workspace)."""
    s, B, Lq, Lk = _indexer_struct(q, k, w, None, None)
    dev = q.device
    if idx is None or idx.dim() != 3:
        raise ValueError("idx must be int32 [B, Lq, k]")
    kk = idx.shape[-1]
    _meta(idx, "idx", (torch.int32,), (B, Lq, kk))
    _meta(pbar, "pbar", (torch.float32,), (B, Lq, kk))
    _placed(dev, idx=idx, pbar=pbar)
    with _alloc_on(stream):
        loss = torch.empty((B, Lq), dtype=torch.float32, device=dev)
        dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
        dw = torch.empty(w.shape, dtype=torch.float32, device=dev)
        if dk is None:
            dk = torch.zeros(k.shape, dtype=torch.float32, device=dev)
    _expect(dk, "dk", (torch.float32,), tuple(k.shape), dev)
    ws = ws or Workspace()
    buf, nbytes = ws.get(workspace_size(DSA_OP_INDEXER_KL, DSA_BF16, B, Lq, Lk, kk), dev, stream)
    _check("dsa_indexer_kl_backward", load_library().dsa_indexer_kl_backward(
        ctypes.byref(s), B, Lq, Lk, _ptr(idx), kk, _ptr(pbar), _ptr(loss), _ptr(dq), _ptr(dw), _ptr(dk),
        _ptr(buf), nbytes, _stream(stream)))
    return {"loss": loss, "dq": dq, "dw": dw, "dk": dk}
