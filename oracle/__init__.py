"""Plain CPU oracle for the DSA lightning-indexer -> top-k -> sparse-attention path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
anything in this package: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

Everything is computed in float64 with numpy, directly from the definitions on
the pages:

* GLM-5.2 技术报告速览：IndexShare 与 critic-based PPO (mloasisblog) -- section
  "IndexShare", the indexer-score equation I_{t,s} = sum_j w_{t,j} ReLU(q_{t,j} . k_s)
  over causal s <= t, followed by a top-k with k = 2048; Full layers run the
  indexer, Shared layers inherit the index set of the nearest Full layer.
* GLM 5.2: Built for Long Horizon Tasks (papers.chlience.com) -- section 5.2
  (FSSS pattern, Shared layers read their own KV), and the discussion section
  "DSA 与 IndexShare 的组合数据流" (sparse core attention recomputes score,
  softmax and value aggregation on the selected positions only; only the top-k
  position IDs flow across layers).
* GLM-5 technical report (Chinese translation), section 3.2 "Reasoning RL",
  paragraph "DSA RL 要点" (the top-k operator must be deterministic).

Pins: every function here is checked by the ``-m "not gpu"`` tests against
hand-worked examples, closed forms, invariants and library routines (see
``tests/test_oracle_*.py``).  No function in this package is "parity unpinned".
"""

from .formats import decode_bf16, decode_e4m3, encode_e4m3, quantize_e4m3_per_token, E4M3_MAX
from .dsa import (
    causal_position,
    indexer_scores,
    indexer_scores_rows,
    topk_row,
    topk_rows,
    sparse_attention_rows,
    layer_group,
)
from .schedule import indexer_types, anchors
from .projections import linear, indexer_projections
from .objective import attention_centroid_rows, indexer_kl_rows
from .accounting import (
    causal_pairs,
    selected_pairs,
    indexer_flops,
    attention_flops,
    cost_model,
)

__all__ = [
    "decode_bf16", "decode_e4m3", "E4M3_MAX",
    "causal_position", "indexer_scores", "indexer_scores_rows", "topk_row", "topk_rows",
    "sparse_attention_rows", "layer_group",
    "causal_pairs", "selected_pairs", "indexer_flops", "attention_flops", "cost_model",
    "linear", "indexer_projections", "attention_centroid_rows", "indexer_kl_rows",
]
