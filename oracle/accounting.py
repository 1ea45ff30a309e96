"""Work accounting for the path (test infrastructure only).

GLM 5.2: Built for Long Horizon Tasks, discussion section "DSA 复杂度的直观含义":
in prefill query i scores about i earlier positions, so the indexer handles
sum_{i=1..L} i candidate pairs, while the core attention handles about L*k selected
pairs; at L = 1e6 and k = 2048 that is about 5e11 and 2.05e9 pairs.
Discussion section "DSA 与 IndexShare 的组合数据流", cost equations:
T_DSA ~ N C_I L^2 + N C_A L k and T_IndexShare ~ r N C_I L^2 + N C_A L k.
"""


def causal_pairs(L, Lq=None):
    """Number of (query, key) pairs with s <= p_i for the last Lq of L positions."""
    Lq = L if Lq is None else Lq
    first = L - Lq + 1                 # keys seen by query 0
    last = L                           # keys seen by the last query
    return (first + last) * Lq // 2


def selected_pairs(L, k, Lq=None):
    """sum over queries of min(k, p_i + 1): pairs the sparse attention reads."""
    Lq = L if Lq is None else Lq
    total = 0
    lo = L - Lq + 1                    # p_0 + 1
    # queries whose causal count is <= k contribute their count, the rest contribute k
    hi_small = min(L, k)
    if lo <= hi_small:
        total += (lo + hi_small) * (hi_small - lo + 1) // 2
        n_big = L - hi_small
    else:
        n_big = Lq
    total += n_big * k
    return total


def indexer_flops(pairs, H_I, d_I):
    """2 * H_I * d_I flops per scored pair (the q.k dot products of every head)."""
    return 2 * H_I * d_I * pairs


def attention_flops(pairs, H, Dqk, Dv):
    """2 * H * (Dqk + Dv) flops per selected pair (QK^T plus PV)."""
    return 2 * H * (Dqk + Dv) * pairs


def cost_model(N, L, k, C_I, C_A, r):
    """(T_DSA, T_IndexShare) of the cost equations for N layers, Full-layer fraction r."""
    t_dsa = N * C_I * L * L + N * C_A * L * k
    t_is = r * N * C_I * L * L + N * C_A * L * k
    return t_dsa, t_is
