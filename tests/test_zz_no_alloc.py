"""dsa_sparse_attn_noalloc (for callers that cannot allocate device memory) against
dsa_sparse_attn: the same kernels, so the outputs must be bit-identical.  Two calls in a row
on the library's buffer, the second with a smaller input, then a prefill-sized call that
needs no buffer; outputs start poisoned so that every element must be written."""
import numpy as np
import pytest
import torch

import synth
import dsa_lightning_indexer_scores_amd as dsa
from tests._helpers import poisoned, all_written

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(B, Lq, Lk, k, seed, mtp=False):
    cfg = synth.get_config("decode200k", L=Lk, B=B)
    lay = synth.attention_inputs(cfg, layer=1, device=DEV, Lq=Lq)
    rng = np.random.default_rng(seed)
    rows = 1 if mtp else Lq
    idx = np.stack([np.sort(rng.permutation(Lk)[:k]) for _ in range(B * rows)]).reshape(B, rows, k)
    idx = idx.astype(np.int32)
    idx[0, 0, ::11] = -1
    return lay, torch.from_numpy(idx).to(DEV)


def _compare(lay, idx, idx_q_stride=None):
    B, Lq, H = lay["q"].shape[:3]
    ref, ref_lse = dsa.sparse_attn(lay, idx, idx_q_stride=idx_q_stride, return_lse=True, ws=dsa.Workspace(),
                                   out=poisoned((B, Lq, H, 512), torch.bfloat16))
    out = poisoned((B, Lq, H, 512), torch.bfloat16)
    lse = poisoned((B, Lq, H), torch.float32)
    dsa.sparse_attn_noalloc(lay, idx, out, lse=lse, idx_q_stride=idx_q_stride)
    torch.cuda.synchronize()
    assert all_written(out) and all_written(ref)
    assert torch.equal(out, ref)
    assert torch.equal(torch.isneginf(lse), torch.isneginf(ref_lse))
    fin = torch.isfinite(ref_lse)
    assert torch.equal(lse[fin], ref_lse[fin])


def test_noalloc_equals_sparse_attn_on_consecutive_calls():
    need = [dsa.workspace_size(dsa.DSA_OP_SPARSE_ATTN, dsa.DSA_BF16, B, 1, Lk, k, 32)
            for B, Lk, k in ((64, 9000, 2048), (3, 2500, 700))]
    assert all(n > 0 for n in need), "both calls must use the split buffer"
    _compare(*_case(64, 1, 9000, 2048, 0))       # decode shape: 64 sequences, keys split
    _compare(*_case(3, 1, 2500, 700, 1))         # a smaller call right after it
    lay, idx = _case(5, 4, 3000, 2048, 2, mtp=True)
    _compare(lay, idx, idx_q_stride=0)           # MTP draft queries sharing one row
    lay, idx = _case(1, 1100, 1100, 256, 3)
    assert dsa.workspace_size(dsa.DSA_OP_SPARSE_ATTN, dsa.DSA_BF16, 1, 1100, 1100, 256, 32) == 0
    _compare(lay, idx)                           # prefill shape: no buffer needed
