"""Pins for oracle/sizing.py against the numbers the pages print."""

from fractions import Fraction

import pytest

from conftest import golden
from oracle import sizing as Z


def test_kv_bytes_per_token_and_sequence():
    g = golden("sizing.json")
    k = g["kv_per_token"]
    per_tok = Z.kv_bytes_per_token(k["layers"], k["kv_heads"], k["d_head"], k["elem_bytes"])
    assert per_tok == k["bytes"] == 128 * 1024
    s = g["sequence_4096"]
    total = Z.sequence_kv_bytes(s["tokens"], k["layers"], k["kv_heads"], k["d_head"], k["elem_bytes"])
    assert total == s["bytes"] and total == s["mib"] * 2 ** 20


def test_block_table_footprint():
    b = golden("sizing.json")["block_table_4096"]
    assert Z.blocks_needed(b["tokens"], b["block_size"]) == b["blocks"]
    assert Z.block_table_bytes(b["tokens"], b["block_size"]) == b["bytes"]
    assert Z.table_to_payload_ratio(b["tokens"], b["block_size"], 131072) == Fraction(1, b["ratio_denominator"])
    assert float(Fraction(1, b["ratio_denominator"])) * 100 == pytest.approx(0.0001907, rel=1e-3)


def test_p3_kv_cache_gb():
    g = golden("sizing.json")["kv_cache_gb"]
    v = Z.kv_cache_gb(*g["args"])
    assert v == pytest.approx(17.179869184, rel=1e-12)
    assert round(v) == g["approx_gb"]


@pytest.mark.parametrize("name", ["capacity_16mib", "exercise_1"])
def test_capacity_examples(name):
    g = golden("sizing.json")[name]
    for bs, e in g["by_block_size"].items():
        r = Z.capacity_plan(g["lengths"], int(bs), g["pool_bytes"], g["bytes_per_slot"])
        assert r["pool_slots"] == g["pool_slots"]
        assert r["blocks"] == e["blocks"] and r["slots"] == e["slots"] and r["waste"] == e["waste"]
        assert r["fits"] == e["fits"]
        assert r["memory_bytes"] == e["memory_mib"] * 2 ** 20
        if "waste_pct" in e:
            assert float(r["waste_fraction"]) * 100 == pytest.approx(e["waste_pct"], abs=0.005)
        if "deficit_slots" in e:
            assert r["deficit_slots"] == e["deficit_slots"]
        if "per_request_waste" in e:
            assert [Z.tail_waste(s, int(bs)) for s in g["lengths"]] == e["per_request_waste"]
    if "index_entries_ratio" in g:
        ie = g["index_entries_ratio"]
        b8 = sum(Z.blocks_needed(s, 8) for s in g["lengths"])
        b16 = sum(Z.blocks_needed(s, 16) for s in g["lengths"])
        assert (b8, b16) == (ie["b8"], ie["b16"]) and b8 / b16 == pytest.approx(ie["approx"], abs=0.005)


def test_tail_waste_bound():
    """0 <= ceil(S/B)*B - S <= B - 1 for every S >= 1 ([P1] section 8)."""
    for B in (1, 2, 8, 16, 32, 64):
        for S in range(1, 300):
            w = Z.tail_waste(S, B)
            assert 0 <= w <= B - 1
            assert (w == 0) == (S % B == 0)
