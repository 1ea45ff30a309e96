"""Shared helpers for the tests: torch tensors -> decoded float64 arrays for the oracle,
and the tolerance rules used for parity."""
import numpy as np
import torch

from oracle import decode_bf16, decode_e4m3


def to_f64(t):
    """Exact float64 values of a stored tensor (fp32, bf16, or uint8 OCP E4M3 codes)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy().astype(np.float64)
    if t.dtype == torch.bfloat16:
        return decode_bf16(t.view(torch.int16).numpy().view(np.uint16))
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return decode_e4m3(t.view(torch.uint8).numpy())
    raise TypeError(t.dtype)


def indexer_to_oracle(ind):
    """Synthetic indexer dict (torch) -> dict of float64 arrays for oracle calls."""
    out = {"q": to_f64(ind["q"]), "k": to_f64(ind["k"]), "w": to_f64(ind["w"])}
    out["q_scale"] = None if ind["q_scale"] is None else to_f64(ind["q_scale"])
    out["k_scale"] = None if ind["k_scale"] is None else to_f64(ind["k_scale"])
    return out


def attn_to_oracle(lay):
    """Synthetic attention dict (torch) -> oracle layer dict (float64)."""
    if "kv" in lay:
        kv = to_f64(lay["kv"])                      # [B, Lk, 576]
        if lay.get("kv_scale") is not None:         # E4M3 codes times their row's scale
            kv = kv * to_f64(lay["kv_scale"])[..., None]
        k = kv[:, :, None, :]                       # Hkv = 1, K = whole latent row
        v = kv[:, :, None, : lay["Dv"]]             # V = first Dv dims
        return {"q": to_f64(lay["q"]), "k": k, "v": v, "sm_scale": lay["sm_scale"], "Hkv": 1}
    return {"q": to_f64(lay["q"]), "k": to_f64(lay["k"]), "v": to_f64(lay["v"]),
            "sm_scale": lay["sm_scale"], "Hkv": lay["Hkv"]}


def index_sets_agree(gpu_idx, ora_idx, ora_scores, n_valid, k, tau):
    """Tolerance rule for index sets: the sets may differ only on positions whose oracle
    score lies within tau*|theta| of the row's k-th oracle score theta; sizes are exact.
    Returns (ok, n_rows_differing, worst_message)."""
    bad = 0
    msg = ""
    for r in range(gpu_idx.shape[0]):
        g = gpu_idx[r]
        o = ora_idx[r]
        gv = set(g[g >= 0].tolist())
        ov = set(o[o >= 0].tolist())
        want = min(k, int(n_valid[r]))
        if len(gv) != want or len(g[g >= 0]) != want:
            return False, r, f"row {r}: size {len(gv)} != {want}"
        if np.any(np.diff(g[g >= 0]) <= 0):
            return False, r, f"row {r}: not ascending"
        if np.any(g[want:] != -1):
            return False, r, f"row {r}: bad padding"
        if gv == ov:
            continue
        sc = ora_scores[r]
        theta = np.sort(sc[: int(n_valid[r])])[::-1][k - 1]
        band = tau * abs(theta)
        for s in gv.symmetric_difference(ov):
            if abs(sc[s] - theta) > band:
                return False, r, f"row {r}: position {s} score {sc[s]} outside band of theta {theta}"
        bad += 1
    return True, bad, msg


def poisoned(shape, dtype, device="cuda"):
    """An output buffer filled with a value no kernel writes (NaN for floats, 0x7F7F7F7F for
    index rows), so that a test can check that every element was written."""
    if dtype == torch.int32:
        return torch.full(shape, 0x7F7F7F7F, dtype=torch.int32, device=device)
    return torch.full(shape, float("nan"), dtype=dtype, device=device)


def all_written(t):
    if t.dtype == torch.int32:
        return not bool((t == 0x7F7F7F7F).any())
    return not bool(torch.isnan(t).any())
