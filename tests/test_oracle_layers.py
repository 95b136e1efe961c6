"""Pin for the oracle's layer predicate: the hand-written golden list."""

import os

from oracle.layers import EXCLUDE_PATTERN, layer_is_quantized

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "exclude_pattern_layers.txt")


def load_golden():
    rows = []
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.rstrip("\n")
            if line.startswith("#"):
                continue
            name, flag = line.split("\t")
            rows.append((name, flag == "1"))
    return rows


def test_pattern_is_the_printed_one():
    assert EXCLUDE_PATTERN == r"^(?!.*(embedder|norm_out|proj_out|to_add_out|to_added_qkv|stream)).*"


def test_golden_layer_names():
    rows = load_golden()
    assert len(rows) >= 25
    for name, want in rows:
        assert layer_is_quantized(name) == want, name


def test_substring_reading():
    subs = ["embedder", "norm_out", "proj_out", "to_add_out", "to_added_qkv", "stream"]
    for name, want in load_golden():
        assert want == (not any(s in name for s in subs)), name
