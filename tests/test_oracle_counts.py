"""Pins of the oracle's count functions against numbers the pages print."""
import json
import os

import pytest

from oracle import counts

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_cache_counts.jsonl")


def _entries():
    with open(GOLDEN) as f:
        return [json.loads(line) for line in f if line.strip()]


@pytest.mark.parametrize("e", _entries(), ids=lambda e: e["id"])
def test_printed_kv_cache_sizes(e):
    a = e["args"]
    got = counts.kv_cache_bytes(a["length"], a["kv_heads"], a["head_dim"], a["elt_bytes"],
                                layers=a["layers"], batch=a["batch"])
    if "expect" in e:
        assert got == e["expect"], e["cite"]
    elif "loose_rel" in e:
        assert abs(got / e["unit"] - e["printed"]) <= e["loose_rel"] * e["printed"], e["cite"]
    else:
        unit_last = 10.0 ** (-e["digits"])
        slack = e.get("slack_units", 0) * unit_last
        assert abs(round(got / e["unit"], e["digits"]) - e["printed"]) <= slack + 1e-9, e["cite"]


def test_cache_elements_proportional_to_kv_heads():
    """The cache element count holds no query-head term: 8 KV heads -> 1 gives exactly 1/8."""
    assert counts.kv_cache_elems(4096, 8, 128, layers=80) == 8 * counts.kv_cache_elems(4096, 1, 128, layers=80)
    assert counts.kv_cache_elems(1, 1, 1) == 2  # K and V


def test_attention_multiplications_have_no_group_term():
    """Scores and weighted sum: h*n*n*d each, the same for every KV-head count."""
    m = counts.attention_mults(64, 2048, 128)
    assert m["scores"] == m["weighted_sum"] == 64 * 2048 * 2048 * 128
    p8 = counts.kv_projection_mults(2048, 8192, 8, 128)
    p1 = counts.kv_projection_mults(2048, 8192, 1, 128)
    assert p8["k_proj"] == 8 * p1["k_proj"]


@pytest.mark.parametrize("hkv", [64, 16, 8, 4, 1])
def test_decode_flops_independent_of_kv_heads(hkv):
    assert counts.decode_flops([2048] * 16, 64, 128) == 1073741824


def test_decode_bytes_scale_with_kv_heads():
    seq = [2048] * 16
    by = {h: counts.decode_bytes(seq, 64, h, 128, 2) for h in (64, 16, 8, 4, 1)}
    qo = 2 * 16 * 64 * 128 * 2
    for h in by:
        assert by[h] - qo == (h * (by[1] - qo))


def test_prefill_pairs():
    assert counts.prefill_pairs(1, True) == 1
    assert counts.prefill_pairs(3, True) == 6 and counts.prefill_pairs(3, False) == 9
    # brute count of the unmasked (i, j) pairs
    assert counts.prefill_pairs(37, True) == sum(1 for i in range(37) for j in range(37) if j <= i)
