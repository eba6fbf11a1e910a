"""Golden fixtures: numbers printed on the pages, expected values from the
oracle (tests/golden/make_golden.py); each fixture carries its citation."""
import json
import os

import oracle

HERE = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(HERE, name), encoding="utf-8") as f:
        return json.load(f)


def test_paging_example_waste_is_confined_to_the_last_page():
    g = _load("paging_example.json")
    i, e = g["inputs"], g["expected"]
    assert e["contiguous_utilisation"] == i["tokens"] / i["reserved"]
    assert e["paged_utilisation"] == oracle.paged_utilisation([i["tokens"]])
    assert 0 <= e["paged_waste_slots"] < i["page_tokens"]
    assert e["paged_slots"] == e["paged_blocks"] * i["page_tokens"]
    assert e["paged_utilisation"] == i["tokens"] / e["paged_slots"]


def test_kv_size_formula_example():
    g = _load("kv_size_example.json")
    i = g["inputs"]
    got = oracle.kv_cache_bytes(i["batch"], i["seq_len"], i["layers"], i["width"], i["elem_bytes"])
    assert got == g["expected"]["bytes"] == 1 << 30
