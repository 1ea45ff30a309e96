"""Pins of the oracle's layer schedule (GLM 5.2: Built for Long Horizon Tasks, section
5.2; GLM-5.2 技术报告速览, section "IndexShare")."""
import json
import os

import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "indexshare_config.json")


def _cfg():
    with open(GOLDEN) as f:
        return json.load(f)


def test_one_group_is_the_fsss_pattern():
    # the group pattern the pages print: full, shared, shared, shared
    cfg = _cfg()
    assert oracle.indexer_types(4, freq=cfg["index_topk_freq"]) == cfg["group_pattern"]


def test_released_config_repeats_fsss_after_the_offset():
    cfg = _cfg()
    freq, off = cfg["index_topk_freq"], cfg["index_skip_topk_offset"]
    types = oracle.indexer_types(80, freq=freq, offset=off)
    period = cfg["group_pattern"]
    assert all(t == period[(l - off) % freq] for l, t in enumerate(types) if l >= off)
    assert types[:off] == ["full"] * off          # the reading of the leading layers
    assert sum(t == "full" for t in types) == off + 20   # 77 periodic layers: 20 groups started


def test_twenty_groups_of_four_have_a_quarter_full():
    # r = 1/4 for the fixed FSSS pattern; 80 layers = 20 groups
    types = oracle.indexer_types(80, freq=4, offset=0)
    assert sum(t == "full" for t in types) == 20
    assert [l for l, t in enumerate(types) if t == "full"] == list(range(0, 80, 4))


def test_shared_layers_use_the_nearest_full_layer_before_them():
    types = oracle.indexer_types(11, freq=4, offset=3)
    # F F F | F S S S | F S S S
    assert types == ["full"] * 4 + ["shared"] * 3 + ["full"] + ["shared"] * 3
    assert oracle.anchors(types) == [0, 1, 2, 3, 3, 3, 3, 7, 7, 7, 7]


def test_explicit_pattern_and_freq_one():
    assert oracle.anchors(oracle.indexer_types(5, pattern="FSFSS")) == [0, 0, 2, 2, 2]
    assert oracle.indexer_types(3, freq=1) == ["full"] * 3      # every layer runs its indexer
    assert oracle.indexer_types(0) == []


@pytest.mark.parametrize("kw", [dict(pattern="FSX"), dict(pattern="FS"), dict(freq=0), dict(offset=-1)])
def test_invalid_schedules_raise(kw):
    with pytest.raises(ValueError):
        oracle.indexer_types(3, **kw)


def test_shared_first_has_no_anchor():
    with pytest.raises(ValueError):
        oracle.anchors(oracle.indexer_types(2, pattern="SF"))
