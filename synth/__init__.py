"""Seeded synthetic inputs for the DSA indexer / top-k / sparse-attention path.

This module only produces inputs (random draws, the per-token FP8 encoding of the
indexer operands, planted heavy keys).  It holds none of the method's arithmetic and
serves both the HIP path and the CPU oracle, which import nothing from each other.

Workloads (shapes of the pages' 100K-1M-context prefill and 200K decode; the pages
name no dataset for this path, so every tensor is a seeded random draw):

* tiny        L=1024, indexer H_I=4, d_I=32 fp32, q^I,k^I ~ N(0, 1/d_I), w ~ U(0,1)/H_I,
              k=64, sparse MHA with 4 heads of d=64 fp32, q,k,v ~ N(0,1).
* prefill16k  L=16384, indexer H_I=64, d_I=128 bf16 (round-to-nearest-even of N(0,1)),
              w ~ U(0,1)/64, k=2048, MLA 32 q-heads over a 576-d latent KV (512 value
              dims + 64 RoPE dims) bf16 N(0,1), 5% of key positions planted with 3x norm.
* prefill128k L=131072, as above but q^I/k^I are OCP FP8 E4M3 with a per-token fp32
              scale amax/448.
* decode200k  64 sequences, 200000 cached keys + 1 new token each (Lk = 200001, Lq = 1),
              FP8 indexer keys, bf16 latent KV; the MTP-draft variant has Lq = 4 queries
              sharing the first query's index set.
* chunk1m     4096-query chunks against up to 1,048,576 FP8 indexer keys.
"""

from dataclasses import dataclass, field
import math

import torch

__all__ = ["Config", "CONFIGS", "get_config", "planted_mask", "indexer_inputs",
           "attention_inputs", "encode_e4m3_per_token"]


@dataclass(frozen=True)
class Config:
    name: str
    L: int                    # keys per sequence (Lk)
    Lq: int                   # queries per sequence
    B: int                    # sequences
    H_I: int
    d_I: int
    idx_dtype: str            # "f32" | "bf16" | "fp8"
    topk: int
    attn: str                 # "mha" | "mla"
    H: int                    # attention query heads
    Hkv: int
    Dqk: int
    Dv: int
    attn_dtype: str           # "f32" | "bf16"
    n_layers: int = 4         # 1 Full + 3 Shared
    planted_frac: float = 0.0
    planted_gain: float = 3.0
    q_std: float = 1.0        # std of the indexer q/k draws
    chunk: int = 0            # query chunk (chunked prefill)
    mtp: int = 1              # queries sharing one index row in the MTP-draft variant
    seed: int = 0
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def sm_scale(self):
        return 1.0 / math.sqrt(self.Dqk)


CONFIGS = {
    "tiny": Config("tiny", L=1024, Lq=1024, B=1, H_I=4, d_I=32, idx_dtype="f32", topk=64,
                   attn="mha", H=4, Hkv=4, Dqk=64, Dv=64, attn_dtype="f32",
                   q_std=1.0 / math.sqrt(32), seed=0),
    "prefill16k": Config("prefill16k", L=16384, Lq=16384, B=1, H_I=64, d_I=128, idx_dtype="bf16",
                         topk=2048, attn="mla", H=32, Hkv=1, Dqk=576, Dv=512, attn_dtype="bf16",
                         planted_frac=0.05, seed=1),
    "prefill128k": Config("prefill128k", L=131072, Lq=131072, B=1, H_I=64, d_I=128, idx_dtype="fp8",
                          topk=2048, attn="mla", H=32, Hkv=1, Dqk=576, Dv=512, attn_dtype="bf16",
                          planted_frac=0.05, seed=2),
    "decode200k": Config("decode200k", L=200001, Lq=1, B=64, H_I=64, d_I=128, idx_dtype="fp8",
                         topk=2048, attn="mla", H=32, Hkv=1, Dqk=576, Dv=512, attn_dtype="bf16",
                         planted_frac=0.05, mtp=4, seed=3),
    "chunk1m": Config("chunk1m", L=1048576, Lq=4096, B=1, H_I=64, d_I=128, idx_dtype="fp8",
                      topk=2048, attn="mla", H=32, Hkv=1, Dqk=576, Dv=512, attn_dtype="bf16",
                      planted_frac=0.05, chunk=4096, seed=4),
}


def get_config(name, **overrides):
    """Named workload, optionally with fields replaced (e.g. a smaller L for tests)."""
    from dataclasses import replace
    return replace(CONFIGS[name], **overrides)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def planted_mask(L, frac, seed, device="cpu"):
    """Boolean [L]: a seeded subset of round(frac*L) key positions (shared by all layers)."""
    m = torch.zeros(L, dtype=torch.bool, device=device)
    n = int(round(frac * L))
    if n > 0:
        g = _gen("cpu", seed * 7919 + 17)
        pos = torch.randperm(L, generator=g)[:n]
        m[pos.to(device)] = True
    return m


def encode_e4m3_per_token(x):
    """x: float32 [T, ...] -> (uint8 OCP E4M3 codes [T, ...], float32 scale [T]) with
    scale = amax/448 per token (1 for an all-zero token); codes = RNE(x / scale)."""
    T = x.shape[0]
    amax = x.reshape(T, -1).abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    y = x / scale.reshape((T,) + (1,) * (x.dim() - 1))
    codes = y.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.to(torch.float32)


def fp8_latent(layer, chunk_rows=1 << 20):
    """A copy of an MLA layer dict whose latent cache is stored as OCP E4M3 codes with one
    fp32 scale per row (amax/448, the encoding of encode_e4m3_per_token), encoded from
    the layer's bf16 rows in row chunks."""
    kv = layer["kv"]
    B, Lk, D = kv.shape
    flat = kv.reshape(B * Lk, D)
    codes = torch.empty((B * Lk, D), dtype=torch.uint8, device=kv.device)
    scales = torch.empty(B * Lk, dtype=torch.float32, device=kv.device)
    for r0 in range(0, B * Lk, chunk_rows):
        c, sc = encode_e4m3_per_token(flat[r0:r0 + chunk_rows].float())
        codes[r0:r0 + chunk_rows] = c
        scales[r0:r0 + chunk_rows] = sc
    out = dict(layer)
    out["kv"] = codes.reshape(B, Lk, D)
    out["kv_scale"] = scales.reshape(B, Lk)
    return out


def _randn_rows(g, shape, device, std, dtype_out, chunk_rows=8192, gain_rows=None, gain=1.0):
    """Draw N(0, std^2) in row chunks (bounded temporaries), optionally scaling planted rows."""
    T = shape[0]
    out = torch.empty(shape, dtype=dtype_out, device=device)
    for r0 in range(0, T, chunk_rows):
        r1 = min(T, r0 + chunk_rows)
        x = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device,
                        dtype=torch.float32) * std
        if gain_rows is not None:
            sel = gain_rows[r0:r1]
            if bool(sel.any()):
                x[sel] *= gain
        out[r0:r1] = x.to(dtype_out)
    return out


def indexer_inputs(cfg, device="cpu", Lq=None, Lk=None, B=None, seed=None, layer=0):
    """Indexer operands of one Full layer.

    Returns dict with q [B,Lq,H_I,d_I], k [B,Lk,d_I] (float32 / bfloat16 / uint8 E4M3
    codes), q_scale [B,Lq] and k_scale [B,Lk] float32 (fp8 only, else None),
    w [B,Lq,H_I] float32, and "dtype" in {"f32","bf16","fp8"}.
    """
    Lq = cfg.Lq if Lq is None else Lq
    Lk = cfg.L if Lk is None else Lk
    B = cfg.B if B is None else B
    seed = cfg.seed if seed is None else seed
    g = _gen(device, seed * 1000 + 101 + layer)
    plant = planted_mask(Lk, cfg.planted_frac, seed, device) if cfg.planted_frac > 0 else None
    qs, ks, ws, qsc, ksc = [], [], [], [], []
    for b in range(B):
        qf = _randn_rows(g, (Lq, cfg.H_I, cfg.d_I), device, cfg.q_std, torch.float32)
        kf = _randn_rows(g, (Lk, cfg.d_I), device, cfg.q_std, torch.float32,
                         gain_rows=plant, gain=cfg.planted_gain)
        w = torch.rand((Lq, cfg.H_I), generator=g, device=device, dtype=torch.float32) / cfg.H_I
        if cfg.idx_dtype == "f32":
            qs.append(qf); ks.append(kf)
        elif cfg.idx_dtype == "bf16":
            qs.append(qf.to(torch.bfloat16)); ks.append(kf.to(torch.bfloat16))
        elif cfg.idx_dtype == "fp8":
            qc, qscale = encode_e4m3_per_token(qf)
            kc, kscale = encode_e4m3_per_token(kf)
            qs.append(qc); ks.append(kc); qsc.append(qscale); ksc.append(kscale)
        else:
            raise ValueError(cfg.idx_dtype)
        ws.append(w)
        del qf, kf
    out = {"q": torch.stack(qs), "k": torch.stack(ks), "w": torch.stack(ws),
           "q_scale": torch.stack(qsc) if qsc else None,
           "k_scale": torch.stack(ksc) if ksc else None,
           "dtype": cfg.idx_dtype, "H_I": cfg.H_I, "d_I": cfg.d_I}
    return out


def attention_inputs(cfg, layer, device="cpu", Lq=None, Lk=None, B=None, seed=None):
    """Sparse-attention operands of one layer of the group.

    MLA: q [B,Lq,H,576], kv [B,Lk,576] (k = kv, v = first 512 dims of kv).
    MHA: q [B,Lq,H,D], k [B,Lk,Hkv,D], v [B,Lk,Hkv,Dv].
    """
    Lq = cfg.Lq if Lq is None else Lq
    Lk = cfg.L if Lk is None else Lk
    B = cfg.B if B is None else B
    seed = cfg.seed if seed is None else seed
    g = _gen(device, seed * 1000 + 503 + 11 * layer)
    dt = torch.float32 if cfg.attn_dtype == "f32" else torch.bfloat16
    plant = planted_mask(Lk, cfg.planted_frac, seed, device) if cfg.planted_frac > 0 else None
    qs, ks, vs = [], [], []
    for b in range(B):
        qs.append(_randn_rows(g, (Lq, cfg.H, cfg.Dqk), device, 1.0, dt))
        if cfg.attn == "mla":
            ks.append(_randn_rows(g, (Lk, cfg.Dqk), device, 1.0, dt,
                                  gain_rows=plant, gain=cfg.planted_gain))
        else:
            ks.append(_randn_rows(g, (Lk, cfg.Hkv, cfg.Dqk), device, 1.0, dt,
                                  gain_rows=plant, gain=cfg.planted_gain))
            vs.append(_randn_rows(g, (Lk, cfg.Hkv, cfg.Dv), device, 1.0, dt))
    out = {"q": torch.stack(qs), "attn": cfg.attn, "H": cfg.H, "Hkv": cfg.Hkv,
           "Dqk": cfg.Dqk, "Dv": cfg.Dv, "sm_scale": cfg.sm_scale, "dtype": cfg.attn_dtype}
    if cfg.attn == "mla":
        out["kv"] = torch.stack(ks)
    else:
        out["k"] = torch.stack(ks)
        out["v"] = torch.stack(vs)
    return out
