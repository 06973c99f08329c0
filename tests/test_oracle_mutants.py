"""Plant plausible mistakes in copies of the oracle and check the pins catch them.

Each mutant is a textual edit of ``oracle/gqa_oracle.c`` compiled into a
temporary library; the pins below (brute force, closed forms, special cases)
must reject every one.  The shipped oracle must pass the same pins.
"""
import math
import os
import subprocess

import numpy as np
import pytest

import gqa_inputs as gi
from oracle import brute, reference as orc
from tests.helpers import to_lists, widen

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "gqa_oracle.c")

MUTANTS = {
    "group_index_modulo": ("const int64_t g = h / gsize; /* contiguous groups */",
                           "const int64_t g = h % Hkv;"),
    "softmax_sign": ("w[j] = exp(w[j] - m);", "w[j] = exp(m - w[j]);"),
    "scale_dropped": ("w[j] = dot * scale;", "w[j] = dot;"),
    "length_off_by_one": ("const int64_t n = seqlens[b];\n                orc_attend",
                          "const int64_t n = seqlens[b] - 1;\n                orc_attend"),
    "row_stride_wrong": ("const int64_t kr = kv0 + j * stride;", "const int64_t kr = kv0 + j * d;"),
    "normalised_by_count": ("out[c] = acc[c] / z;", "out[c] = acc[c] / (double)n;"),
    "causal_off_by_one": ("const int64_t n = causal ? pos + 1 : P;",
                          "const int64_t n = causal ? pos : P;"),
    "v_read_from_k": ("acc[c] += w[j] * orc_elem(v, vr + c, dtype);",
                      "acc[c] += w[j] * orc_elem(k, vr + c, dtype);"),
    "max_not_updated": ("if (w[j] > m)\n            m = w[j];", "if (w[j] > m)\n            m = m;"),
    "query_row_of_wrong_head": ("orc_attend(q, (b * Hq + h) * d, k, v, ((b * Lmax) * Hkv + g) * d,\n",
                                "orc_attend(q, (b * Hq + g) * d, k, v, ((b * Lmax) * Hkv + g) * d,\n"),
}


def _pins():
    """Run a compact set of pins against the currently loaded oracle; return failures."""
    failed = []

    c = gi.decode_case(2, 8, 2, 8, 7, [7, 3], "bf16", q_seed=5, kv_seed=6)
    try:
        got = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
        ref = np.array(brute.decode(to_lists(c.q), to_lists(c.k), to_lists(c.v), [7, 3], c.scale))
        if not np.allclose(got, ref, rtol=1e-12, atol=1e-12):
            failed.append("brute_decode")
    except orc.OracleError:
        failed.append("brute_decode_error")

    p = gi.prefill_case(1, 5, 4, 2, 8, "bf16", seed=7)
    got = orc.prefill(p.q, p.k, p.v, True, p.scale)
    ref = np.array(brute.prefill(to_lists(p.q), to_lists(p.k), to_lists(p.v), True, p.scale))
    if not np.allclose(got, ref, rtol=1e-12, atol=1e-12):
        failed.append("brute_prefill")

    m = gi.decode_case(1, 4, 4, 8, 9, [9], "f32", q_seed=8, kv_seed=9)
    if not np.array_equal(orc.decode(m.q, m.k, m.v, m.seqlens, m.scale),
                          orc.mha_decode(m.q, m.k, m.v, m.seqlens, m.scale)):
        failed.append("mha_equality")

    s = gi.decode_case(1, 4, 2, 8, 3, [1], "f32", q_seed=10, kv_seed=11)
    out = orc.decode(s.q, s.k, s.v, s.seqlens, s.scale)
    for h in range(4):
        if not np.array_equal(out[0, h], widen(s.v[0, 0, h // 2])):
            failed.append("single_key")
            break

    u = gi.decode_case(1, 2, 1, 8, 6, [6], "f32", q_seed=12, kv_seed=13)
    out = orc.decode(u.q, u.k, u.v, u.seqlens, 0.0)
    vv = widen(u.v[0, :6, 0])
    mean = np.array([math.fsum(vv[:, col]) / 6 for col in range(8)])
    if not np.allclose(out[0, 0], mean, rtol=1e-14, atol=1e-14):
        failed.append("mean_of_v")
    return failed


@pytest.fixture(scope="module")
def src_text():
    with open(SRC) as f:
        return f.read()


def test_shipped_oracle_passes_compact_pins():
    assert _pins() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, src_text, tmp_path):
    old, new = MUTANTS[name]
    assert src_text.count(old) >= 1, "mutation site not found: %s" % name
    mutated = src_text.replace(old, new)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mutated)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", str(lib), str(csrc), "-lm"], check=True)
    prev = orc.swap_library(str(lib))
    try:
        failed = _pins()
    finally:
        orc.swap_library(None)
        if prev is not None:
            orc._lib = prev
    assert failed, "mutant %s passed every pin" % name
