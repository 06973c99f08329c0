"""The derived per-element bounds (tests/bounds.py) against plausible mistakes.

At full length the stated tolerance (2e-2 + 1e-2 |ref|) admits outputs that
come from a wrong computation: a dropped 32-key step, a 5% softmax scale
error, a piece boundary that loses or repeats a key.  Each such output,
computed with the oracle itself on changed inputs and rounded to bf16 as the
kernel's output is, must pass the stated tolerance (so the stated check
alone cannot see it) and break the derived bound; the correctly rounded
oracle output must stay inside the bound.  Runs on the CPU only.
"""
import numpy as np
import pytest

import gqa_inputs as gi
from oracle import reference as orc
from tests import bounds as bd
from tests.helpers import bf16_tol_ok, widen


def _bf16(x):
    return widen(gi.bf16_bits_from_f32(np.asarray(x, np.float32)))


@pytest.fixture(scope="module")
def layer():
    """Four sequences of the 70B-class layer (Hq 64, Hkv 8, d 128, L 4096)."""
    c = gi.decode_case(4, 64, 8, 128, 4096, [4096] * 4, "bf16", q_seed=2, kv_seed=2, invalid="zero")
    ref, sig, mu, kap, n = bd.decode_terms(c)
    return c, ref, bd.decode_bound(ref, sig, mu, kap, n, 128)


def test_rounded_decode_output_is_inside_the_bound(layer):
    c, ref, bound = layer
    assert bd.assert_within(_bf16(ref), ref, bound, "bf16(oracle)") < 1.0


def _decode_mistake(c, kind):
    sl = c.seqlens
    if kind == "last_32_key_step_dropped":
        return orc.decode(c.q, c.k, c.v, sl - 32, c.scale)
    if kind == "scale_5_percent_high":
        return orc.decode(c.q, c.k, c.v, sl, c.scale * 1.05)
    if kind == "last_key_dropped":
        return orc.decode(c.q, c.k, c.v, sl - 1, c.scale)
    if kind == "piece_boundary_loses_a_key":       # pieces [0, 2047) and [2048, 4096)
        k = np.ascontiguousarray(np.delete(c.k, 2047, axis=1))
        v = np.ascontiguousarray(np.delete(c.v, 2047, axis=1))
        return orc.decode(c.q, k, v, sl - 1, c.scale)
    if kind == "piece_boundary_repeats_a_key":     # pieces [0, 2049) and [2048, 4096)
        k = np.ascontiguousarray(np.insert(c.k, 2048, c.k[:, 2048], axis=1))
        v = np.ascontiguousarray(np.insert(c.v, 2048, c.v[:, 2048], axis=1))
        return orc.decode(c.q, k, v, sl + 1, c.scale)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["last_32_key_step_dropped", "scale_5_percent_high", "last_key_dropped",
                                  "piece_boundary_loses_a_key", "piece_boundary_repeats_a_key"])
def test_decode_mistake_passes_stated_tolerance_but_breaks_derived_bound(layer, kind):
    c, ref, bound = layer
    wrong = _bf16(_decode_mistake(c, kind))
    ok, err = bf16_tol_ok(wrong, ref)
    assert ok, "the stated tolerance already rejects %s (max err %.3g)" % (kind, err)
    with pytest.raises(AssertionError):
        bd.assert_within(wrong, ref, bound, kind)


@pytest.fixture(scope="module")
def prompt():
    p = gi.prefill_case(1, 1024, 8, 2, 128, "bf16", seed=5)
    ref, sig, mu, kap, n = bd.prefill_terms(p)
    return p, ref, bd.prefill_bound(ref, sig, mu, kap, n, 128)


def test_rounded_prefill_output_is_inside_the_bound(prompt):
    p, ref, bound = prompt
    assert bd.assert_within(_bf16(ref), ref, bound, "bf16(oracle)") < 1.0


@pytest.mark.parametrize("factor", [1.01, 1.02])
def test_prefill_scale_error_passes_stated_tolerance_but_breaks_derived_bound(prompt, factor):
    p, ref, bound = prompt
    rows = np.s_[:, 768:]
    wrong = _bf16(orc.prefill(p.q, p.k, p.v, True, p.scale * factor))
    ok, err = bf16_tol_ok(wrong[rows], ref[rows])
    assert ok, err
    with pytest.raises(AssertionError):
        bd.assert_within(wrong[rows], ref[rows], bound[rows], "scale x%.2f" % factor)


@pytest.mark.parametrize("kind", ["diagonal_key_dropped", "key_511_lost"])
def test_prefill_lost_key_breaks_derived_bound(prompt, kind):
    p, ref, bound = prompt
    q = np.ascontiguousarray(p.q[:, 768:])
    if kind == "diagonal_key_dropped":   # row i sees keys 0 .. i-1: i-1 is its last position
        wrong = orc.decode_ex(q, p.k, p.v, np.array([1023], np.int32), p.scale)
    else:
        k = np.ascontiguousarray(np.delete(p.k, 511, axis=1))
        v = np.ascontiguousarray(np.delete(p.v, 511, axis=1))
        wrong = orc.decode_ex(q, k, v, np.array([1023], np.int32), p.scale)
    with pytest.raises(AssertionError):
        bd.assert_within(_bf16(wrong), ref[:, 768:], bound[:, 768:], kind)


@pytest.mark.parametrize("kv", ["fp8", "e5m2", "same"])
def test_rounded_extended_output_is_inside_the_bound(kv):
    c = gi.decode_ex_case(4, 4, 64, 8, 128, 1024, [1024, 1000, 777, 64], "bf16", seed=91, kv=kv,
                          window=300)
    ref, sig, mu, kap, n = bd.ex_terms(c)
    bound = bd.decode_bound(ref, sig, mu, kap, n, 128)
    assert bd.assert_within(_bf16(ref), ref, bound, "bf16(oracle)") < 1.0
