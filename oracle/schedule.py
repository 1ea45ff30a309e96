"""Layer schedule of an IndexShare stack (test infrastructure, see the package header).

GLM 5.2: Built for Long Horizon Tasks, section 5.2 "IndexShare / IndexCache for DSA":
the released configuration sets index_topk_freq = 4, index_skip_topk_offset = 3 and
index_topk_pattern = null, and past the offset the indexer types of the layers repeat
full, shared, shared, shared (the fixed FSSS pattern).  GLM-5.2 技术报告速览, section
"IndexShare": a Shared layer uses the index set of the nearest Full layer before it.

The pages do not say what the layers before the offset are.  Reading used here: they
are Full (each runs its own indexer), so the periodic part starts at layer `offset`.
An explicit per-layer pattern ('F' / 'S'), when given, is taken as is.
"""


def indexer_types(n_layers, freq=4, offset=0, pattern=None):
    """'full' / 'shared' for every layer, in layer order."""
    if pattern is not None:
        if len(pattern) != n_layers or any(c not in "FS" for c in pattern):
            raise ValueError("pattern must have one 'F' or 'S' per layer")
        return ["full" if c == "F" else "shared" for c in pattern]
    if freq < 1 or offset < 0 or n_layers < 0:
        raise ValueError("freq >= 1, offset >= 0, n_layers >= 0")
    period = ["full"] + ["shared"] * (freq - 1)
    types = []
    for layer in range(n_layers):
        if layer < offset:
            types.append("full")
        else:
            types.append(period[(layer - offset) % freq])
    return types


def anchors(types):
    """For every layer the Full layer whose index set it attends with."""
    out = []
    current = None
    for layer, t in enumerate(types):
        if t == "full":
            current = layer
        elif current is None:
            raise ValueError("a Shared layer needs a Full layer before it")
        out.append(current)
    return out
