"""Pins of the work accounting against the figures printed on the pages (CPU only)."""
import json
import os

from oracle import causal_pairs, selected_pairs, indexer_flops, attention_flops, cost_model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pair_counts_match_the_pages_figures():
    g = json.load(open(os.path.join(GOLDEN, "pair_counts.json")))
    L, k = g["L"], g["k"]
    cp = causal_pairs(L)
    sp = selected_pairs(L, k)
    # printed to 1 and 3 significant digits respectively
    assert round(cp / 1e11) * 1e11 == g["causal_pairs_approx"]
    assert round(sp / 1e7) * 1e7 == g["selected_pairs_approx"]


def test_closed_forms_on_small_cases():
    # brute force over queries
    for L in (1, 2, 5, 17):
        for Lq in range(1, L + 1):
            n = [L - Lq + 1 + i for i in range(Lq)]
            assert causal_pairs(L, Lq) == sum(n)
            for k in (1, 3, 8, 40):
                assert selected_pairs(L, k, Lq) == sum(min(k, x) for x in n)


def test_flops_and_cost_model():
    assert indexer_flops(10, 64, 128) == 10 * 2 * 64 * 128
    assert attention_flops(3, 32, 576, 512) == 3 * 2 * 32 * 1088
    t_dsa, t_is = cost_model(N=80, L=1000, k=10, C_I=1.0, C_A=0.0, r=0.25)
    assert t_is / t_dsa == 0.25                     # indexer-only: r
    t_dsa, t_is = cost_model(N=80, L=1000, k=10, C_I=0.0, C_A=1.0, r=0.25)
    assert t_is == t_dsa                            # attention cost is not shared
