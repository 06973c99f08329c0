"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: the
separately written pure-Python brute force, closed forms, special cases that
reduce to a simpler method (MHA, MQA), and invariants of the softmax-weighted
average.  No GPU is involved.
"""
import math

import numpy as np
import pytest

import gqa_inputs as gi
from oracle import brute, reference as orc
from tests.helpers import to_lists, widen


def small_decode(B, Hq, Hkv, d, Lmax, seqlens, dtype="f32", seed=7, invalid="nan", scale=None):
    return gi.decode_case(B, Hq, Hkv, d, Lmax, seqlens, dtype, q_seed=seed, kv_seed=seed + 100,
                          invalid=invalid, scale=scale)


def rel_close(a, b, rel):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.all(np.abs(a - b) <= rel * np.maximum(1.0, np.abs(b)))


# --- C10: tiny inputs against the fp64 brute force ------------------------

@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2), (8, 1), (6, 3), (4, 2)])
@pytest.mark.parametrize("d", [4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_matches_brute_force(Hq, Hkv, d, dtype):
    seqlens = [7, 1]
    c = small_decode(2, Hq, Hkv, d, 7, seqlens, dtype=dtype, seed=Hq * 10 + Hkv + d)
    got = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
    ref = brute.decode(to_lists(c.q), to_lists(c.k), to_lists(c.v), seqlens, c.scale)
    assert rel_close(got, ref, 1e-12)


@pytest.mark.parametrize("L", [1, 2, 7])
def test_decode_brute_force_lengths(L):
    c = small_decode(1, 4, 2, 8, 7, [L], seed=L)
    got = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
    ref = brute.decode(to_lists(c.q), to_lists(c.k), to_lists(c.v), [L], c.scale)
    assert rel_close(got, ref, 1e-12)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (4, 1), (4, 4)])
def test_prefill_matches_brute_force(causal, Hq, Hkv):
    c = gi.prefill_case(2, 5, Hq, Hkv, 8, "bf16", seed=11 + Hkv, causal=causal)
    got = orc.prefill(c.q, c.k, c.v, causal, c.scale)
    ref = brute.prefill(to_lists(c.q), to_lists(c.k), to_lists(c.v), causal, c.scale)
    assert rel_close(got, ref, 1e-12)


# --- C1 / C2 / C3: the special cases and the repeat-expanded form ----------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mha_special_case_is_exact(dtype):
    """G = Hq: GQA must equal a separately written MHA exactly (bitwise)."""
    c = small_decode(3, 8, 8, 16, 33, [33, 5, 17], dtype=dtype, seed=21)
    a = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
    b = orc.mha_decode(c.q, c.k, c.v, c.seqlens, c.scale)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mqa_special_case_is_exact(dtype):
    """G = 1: GQA must equal a separately written MQA exactly (bitwise)."""
    c = small_decode(3, 8, 1, 16, 33, [1, 33, 20], dtype=dtype, seed=22)
    a = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
    b = orc.mqa_decode(c.q, c.k, c.v, c.seqlens, c.scale)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (8, 4), (6, 3), (16, 4), (8, 1)])
def test_repeat_expanded_equals_gqa(Hq, Hkv):
    """Expanding each K/V head to its Hq/Hkv query heads, then MHA, is the same computation."""
    c = small_decode(2, Hq, Hkv, 8, 19, [19, 11], dtype="bf16", seed=23 + Hq + Hkv)
    gs = Hq // Hkv
    k_rep = np.ascontiguousarray(np.repeat(c.k, gs, axis=2))
    v_rep = np.ascontiguousarray(np.repeat(c.v, gs, axis=2))
    a = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
    b = orc.mha_decode(c.q, k_rep, v_rep, c.seqlens, c.scale)
    assert np.array_equal(a, b)


def test_groups_are_contiguous_blocks():
    """Query heads 0..gs-1 use KV head 0: perturbing KV head 1 must not change them."""
    Hq, Hkv = 8, 2
    c = small_decode(1, Hq, Hkv, 8, 9, [9], seed=24)
    a = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
    k2 = c.k.copy()
    k2[:, :, 1, :] *= np.float32(-3.0)
    b = orc.decode(c.q, k2, c.v, c.seqlens, c.scale)
    assert np.array_equal(a[:, :4], b[:, :4])
    assert not np.allclose(a[:, 4:], b[:, 4:])


def test_fewer_groups_change_the_output():
    """With the same q, reducing the KV heads changes the result (different K/V)."""
    outs = {}
    for hkv in (8, 2, 1):
        c = gi.tiny_decode(hkv)
        outs[hkv] = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
    assert not np.allclose(outs[8], outs[2]) and not np.allclose(outs[2], outs[1])


# --- C4: softmax rows sum to 1; the output is the weighted sum -------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_weights_sum_to_one(dtype):
    c = small_decode(2, 4, 2, 16, 300, [300, 3], dtype=dtype, seed=25)
    for b in range(2):
        for h in range(4):
            w, out = orc.decode_weights(c.q, c.k, c.v, c.seqlens, c.scale, b, h)
            assert np.all(w > 0)
            assert abs(math.fsum(w) - 1.0) <= 1e-14
            g = h // 2
            vw = widen(c.v[b, : c.seqlens[b], g, :])
            ref = np.array([math.fsum(w * vw[:, col]) for col in range(vw.shape[1])])
            assert rel_close(out, ref, 1e-13)
            full = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
            assert np.array_equal(full[b, h], out)


# --- C5: all-equal keys, or scale 0, give the mean of V ---------------------

@pytest.mark.parametrize("mode", ["equal_keys", "zero_scale"])
def test_uniform_attention_is_mean_of_v(mode):
    c = small_decode(2, 4, 2, 16, 40, [40, 13], seed=26)
    k = c.k.copy()
    scale = c.scale
    if mode == "equal_keys":
        for b in range(2):
            k[b, : c.seqlens[b]] = k[b, 0:1]
    else:
        scale = 0.0
    out = orc.decode(c.q, k, c.v, c.seqlens, scale)
    for b in range(2):
        n = int(c.seqlens[b])
        for h in range(4):
            vv = widen(c.v[b, :n, h // 2, :])
            mean = np.array([math.fsum(vv[:, col]) / n for col in range(vv.shape[1])])
            assert rel_close(out[b, h], mean, 1e-14)


# --- C6: a single cached row returns that row of V exactly ----------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_key_returns_v(dtype):
    c = small_decode(3, 8, 2, 32, 4, [1, 1, 1], dtype=dtype, seed=27)
    out = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
    for b in range(3):
        for h in range(8):
            assert np.array_equal(out[b, h], widen(c.v[b, 0, h // 4]))


def test_zero_length_row_is_zero():
    c = small_decode(2, 4, 2, 8, 5, [0, 5], seed=28)
    out = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
    assert np.all(out[0] == 0.0) and np.all(np.isfinite(out[1]))


# --- two keys: the softmax is a logistic function of the score gap ---------

def test_two_keys_logistic_form():
    c = small_decode(1, 2, 1, 8, 2, [2], seed=29)
    out = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
    q = widen(c.q[0])
    k = widen(c.k[0, :, 0])
    v = widen(c.v[0, :, 0])
    for h in range(2):
        gap = c.scale * (math.fsum(q[h] * k[1]) - math.fsum(q[h] * k[0]))
        w0 = 1.0 / (1.0 + math.exp(gap))
        ref = w0 * v[0] + (1.0 - w0) * v[1]
        assert rel_close(out[0, h], ref, 1e-13)


def test_dominant_key_selects_its_value():
    """A key aligned with q and scaled up takes all the weight."""
    c = small_decode(1, 1, 1, 8, 6, [6], seed=30)
    k = c.k.copy()
    k[0, 3, 0, :] = c.q[0, 0, :] * np.float32(64.0)
    out = orc.decode(c.q, k, c.v, c.seqlens, 1.0)
    assert np.allclose(out[0, 0], widen(c.v[0, 3, 0]), atol=1e-12)


# --- C7: causal prefill row i equals decode over i+1 rows -----------------

def test_causal_prefill_row_equals_decode():
    B, P, Hq, Hkv, d = 2, 9, 4, 2, 8
    c = gi.prefill_case(B, P, Hq, Hkv, d, "bf16", seed=31)
    pre = orc.prefill(c.q, c.k, c.v, True, c.scale)
    for i in range(P):
        q_dec = np.ascontiguousarray(c.q[:, i])
        dec = orc.decode(q_dec, c.k, c.v, np.full(B, i + 1, np.int32), c.scale)
        assert np.array_equal(pre[:, i], dec)


def test_noncausal_prefill_rows_equal_full_decode():
    B, P, Hq, Hkv, d = 1, 6, 4, 1, 8
    c = gi.prefill_case(B, P, Hq, Hkv, d, "f32", seed=32, causal=False)
    pre = orc.prefill(c.q, c.k, c.v, False, c.scale)
    for i in range(P):
        dec = orc.decode(np.ascontiguousarray(c.q[:, i]), c.k, c.v, np.full(B, P, np.int32), c.scale)
        assert np.array_equal(pre[:, i], dec)


# --- C11: permuting cached rows (K and V together) changes nothing --------

def test_permutation_invariance():
    c = small_decode(1, 4, 2, 16, 50, [50], seed=33)
    perm = np.random.default_rng(0).permutation(50)
    k = np.ascontiguousarray(c.k[:, perm])
    v = np.ascontiguousarray(c.v[:, perm])
    a = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
    b = orc.decode(c.q, k, v, c.seqlens, c.scale)
    assert rel_close(a, b, 1e-13)


# --- C12: affine in V ------------------------------------------------------

def test_affine_in_v():
    c = small_decode(1, 4, 2, 8, 20, [20], seed=34)
    # dyadic V so that 2*V + 0.25 is exact in fp32
    v = (np.random.default_rng(1).integers(-16, 16, c.v.shape) / 8.0).astype(np.float32)
    v2 = (2.0 * v + 0.25).astype(np.float32)
    a = orc.decode(c.q, c.k, v, c.seqlens, c.scale)
    b = orc.decode(c.q, c.k, v2, c.seqlens, c.scale)
    assert rel_close(b, 2.0 * a + 0.25, 1e-13)


# --- rows beyond seqlens are never read ------------------------------------

def test_invalid_rows_never_read():
    a = small_decode(2, 8, 2, 16, 64, [10, 64], dtype="bf16", seed=35, invalid="nan")
    b = small_decode(2, 8, 2, 16, 64, [10, 64], dtype="bf16", seed=35, invalid="zero")
    oa = orc.decode(a.q, a.k, a.v, a.seqlens, a.scale)
    ob = orc.decode(b.q, b.k, b.v, b.seqlens, b.scale)
    assert np.all(np.isfinite(oa)) and np.array_equal(oa, ob)


def test_sampled_rows_match_full():
    c = small_decode(3, 8, 2, 16, 30, [30, 2, 17], dtype="bf16", seed=36)
    full = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale)
    rows = np.array([0, 23, 9, 15, 8])
    part = orc.decode(c.q, c.k, c.v, c.seqlens, c.scale, rows=rows)
    assert np.array_equal(part, full.reshape(-1, 16)[rows])


def test_rejects_uneven_groups():
    c = small_decode(1, 6, 3, 8, 4, [4], seed=37)
    bad_k = np.ascontiguousarray(np.concatenate([c.k, c.k[:, :, :1]], axis=2))  # 4 KV heads, Hq=6
    with pytest.raises(orc.OracleError):
        orc.decode(c.q, bad_k, bad_k, c.seqlens, c.scale)
