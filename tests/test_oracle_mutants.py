"""Plant plausible mistakes in copies of the oracle and check the pins catch them.

Each mutant is a textual edit of ``oracle/gqa_oracle.c`` compiled into a
temporary library; the pins below (brute force, closed forms, special cases)
must reject every one.  The shipped oracle must pass the same pins.  Each
mutant runs in a child interpreter: a mutant that indexes out of bounds may
crash, and a crash counts as a failed pin.
"""
import math
import os
import subprocess
import sys

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
    "ex_token_order_reversed": ("const int64_t pos = seqlens[b] - T + t;",
                                "const int64_t pos = seqlens[b] - 1 - t;"),
    "ex_window_off_by_one": ("(window > 0 && pos - window + 1 > 0) ? pos - window + 1 : 0;",
                             "(window > 0 && pos - window > 0) ? pos - window : 0;"),
    "ex_paged_block_index": ("block_table[b * max_blocks + j / bs];",
                             "block_table[b * max_blocks + j % bs];"),
    "ex_e4m3_exponent_bias": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);",
                              "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "ex_v_scale_from_k": ("const double vs = kv_fmt ? (double)v_scale[g] : 1.0;",
                          "const double vs = kv_fmt ? (double)k_scale[g] : 1.0;"),
    "ex_e5m2_exponent_bias": ("v = ldexp(1.0 + (double)m / 4.0, e - 15);",
                              "v = ldexp(1.0 + (double)m / 4.0, e - 16);"),
    "ex_e5m2_mantissa_width": ("v = ldexp(1.0 + (double)m / 4.0, e - 15);",
                               "v = ldexp(1.0 + (double)m / 8.0, e - 15);"),
    "ex_e5m2_read_as_e4m3": ("if (kv_fmt == 2)\n        return oracle_e5m2_value",
                             "if (kv_fmt == 2)\n        return oracle_e4m3_value"),
    "ex_append_row_off_by_one": ("const int64_t j = seqlens[b] - T + t;",
                                 "const int64_t j = seqlens[b] - T + t - 1;"),
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

    # extended decode: brute force with every feature on, prefill rows, append
    import torch
    e = gi.decode_ex_case(2, 3, 4, 2, 8, 12, [12, 6], "bf16", seed=31, kv="fp8", paged=True,
                          block_size=4, window=4)
    try:
        got = orc.decode_ex(e.q, e.k, e.v, e.seqlens, e.scale, k_scale=e.k_scale,
                            v_scale=e.v_scale, block_table=e.block_table,
                            block_size=e.block_size, window=4)

        def w8(codes, sc):
            t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
            return t.to(torch.float64).numpy() * np.asarray(sc, np.float64)[:, None]

        ref = brute.decode_ex(widen(e.q).tolist(), w8(e.k, e.k_scale).tolist(),
                              w8(e.v, e.v_scale).tolist(), e.seqlens.tolist(), e.scale, window=4,
                              block_table=e.block_table.tolist(), block_size=4)
        if not np.allclose(got, np.array(ref), rtol=1e-12, atol=1e-12):
            failed.append("brute_decode_ex")
    except orc.OracleError:
        failed.append("brute_decode_ex_error")
    # E5M2 rows widened through binary16 (an E5M2 code is the top byte of a half)
    e5 = gi.decode_ex_case(2, 2, 4, 2, 8, 10, [10, 5], "bf16", seed=34, kv="e5m2", window=3)
    try:
        got = orc.decode_ex(e5.q, e5.k, e5.v, e5.seqlens, e5.scale, k_scale=e5.k_scale,
                            v_scale=e5.v_scale, window=3, kv_format="e5m2")

        def w5(codes, sc):
            half = (np.ascontiguousarray(codes).astype(np.uint16) << 8).view(np.float16)
            return half.astype(np.float64) * np.asarray(sc, np.float64)[:, None]

        ref = brute.decode_ex(widen(e5.q).tolist(), w5(e5.k, e5.k_scale).tolist(),
                              w5(e5.v, e5.v_scale).tolist(), e5.seqlens.tolist(), e5.scale,
                              window=3)
        if not np.allclose(got, np.array(ref), rtol=1e-12, atol=1e-12):
            failed.append("brute_decode_ex_e5m2")
    except orc.OracleError:
        failed.append("brute_decode_ex_e5m2_error")
    pf = gi.prefill_case(1, 9, 4, 2, 8, "bf16", seed=32)
    try:
        rows = orc.decode_ex(np.ascontiguousarray(pf.q[:, 6:]), pf.k, pf.v, np.array([9], np.int32),
                             pf.scale)
        if not np.array_equal(rows, orc.prefill(pf.q, pf.k, pf.v, True, pf.scale)[:, 6:]):
            failed.append("decode_ex_prefill_rows")
    except orc.OracleError:
        failed.append("decode_ex_prefill_rows_error")
    a = gi.decode_ex_case(2, 2, 4, 2, 8, 8, [8, 5], "bf16", seed=33, paged=True, block_size=4)
    kk, vv2 = a.k_pre.copy(), a.v_pre.copy()
    try:
        orc.append(kk, vv2, a.k_new, a.v_new, a.seqlens, block_table=a.block_table, block_size=4)
        if not (np.array_equal(kk, a.k) and np.array_equal(vv2, a.v)):
            failed.append("append_rows")
    except orc.OracleError:
        failed.append("append_error")

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
    child = ("import sys; from oracle import reference as orc; import tests.test_oracle_mutants as m; "
             "orc.swap_library(sys.argv[1]); f = m._pins(); print(f); sys.exit(3 if f else 0)")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", child, str(lib)], cwd=root, env=env,
                       capture_output=True, text=True, timeout=300)
    # 3: some pin failed; negative: killed by a signal (a crash is a failed pin)
    assert r.returncode == 3 or r.returncode < 0, \
        "mutant %s passed every pin (rc %d): %s %s" % (name, r.returncode, r.stdout, r.stderr[-400:])
