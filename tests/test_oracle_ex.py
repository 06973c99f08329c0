"""Pins of the extended decode oracle (several new tokens, append, sliding
window, paged cache, FP8 E4M3 and E5M2 caches) against things other than
itself: the two formats' definitions and torch's float8 casts, the separately written decode and
prefill oracles, cache slices, closed forms, and the pure-Python brute force.
"""
import os

import numpy as np
import pytest

import gqa_inputs as gi
from oracle import brute, reference as orc
from tests.helpers import widen

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_fp8(fname):
    rows = []
    for line in open(os.path.join(GOLDEN_DIR, fname)):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()[:2]
        if val in ("nan", "inf", "-inf"):
            rows.append((int(code, 16), float(val)))
        else:
            mant, exp = val.split("*2^")
            rows.append((int(code, 16), float(mant) * 2.0 ** int(exp) if mant != "-0" else -0.0))
    return rows


@pytest.mark.parametrize("fname,fn", [("e4m3_values.txt", orc.e4m3_value),
                                      ("e5m2_values.txt", orc.e5m2_value)])
def test_fp8_golden_values(fname, fn):
    for code, val in _golden_fp8(fname):
        got = fn(code)
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def _torch_fp8(fmt):
    torch = pytest.importorskip("torch")
    return torch, {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[fmt]


@pytest.mark.parametrize("fmt,fn", [("e4m3", orc.e4m3_value), ("e5m2", orc.e5m2_value)])
def test_fp8_matches_torch_cast_all_codes(fmt, fn):
    torch, tdt = _torch_fp8(fmt)
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(tdt).to(torch.float64).numpy()
    got = np.array([fn(c) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e5m2_is_the_top_byte_of_a_half():
    """E5M2 shares binary16's sign and exponent fields: code c is the half
    with bits c << 8, for every one of the 256 codes."""
    codes = np.arange(256, dtype=np.uint16)
    ref = (codes << 8).astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([orc.e5m2_value(int(c)) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def _fp8_widen(codes, scale_per_head, fmt="e4m3"):
    """FP8 rows [..., Hkv, d] -> float64 values * per-head scale, via torch's cast."""
    torch, tdt = _torch_fp8(fmt)
    vals = torch.from_numpy(np.ascontiguousarray(codes)).view(tdt).to(torch.float64).numpy()
    return vals * np.asarray(scale_per_head, np.float64)[:, None]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token_equals_decode(dtype):
    c = gi.decode_ex_case(3, 1, 8, 2, 16, 40, [40, 17, 1], dtype, seed=21)
    got = orc.decode_ex(c.q, c.k, c.v, c.seqlens, c.scale)
    ref = orc.decode(np.ascontiguousarray(c.q[:, 0]), c.k, c.v, c.seqlens, c.scale)
    assert np.array_equal(got[:, 0], ref)


@pytest.mark.parametrize("T", [1, 3, 5])
def test_tokens_are_causal_prefill_rows(T):
    p = gi.prefill_case(2, 29, 8, 4, 16, "bf16", seed=22)
    ref = orc.prefill(p.q, p.k, p.v, True, p.scale)
    q = np.ascontiguousarray(p.q[:, 29 - T:])
    got = orc.decode_ex(q, p.k, p.v, np.array([29, 29], np.int32), p.scale)
    assert np.array_equal(got, ref[:, 29 - T:])


def test_window_equals_decode_on_cache_slice():
    W, T = 7, 3
    c = gi.decode_ex_case(2, T, 4, 2, 16, 30, [30, 12], "bf16", seed=23, window=W)
    got = orc.decode_ex(c.q, c.k, c.v, c.seqlens, c.scale, window=W)
    for b in range(2):
        n = int(c.seqlens[b])
        for t in range(T):
            pos = n - T + t
            lo = max(0, pos - W + 1)
            ks = np.ascontiguousarray(c.k[b:b + 1, lo:pos + 1])
            vs = np.ascontiguousarray(c.v[b:b + 1, lo:pos + 1])
            ref = orc.decode(np.ascontiguousarray(c.q[b:b + 1, t]), ks, vs,
                             np.array([pos + 1 - lo], np.int32), c.scale)
            assert np.array_equal(got[b, t], ref[0]), (b, t)


def test_window_wider_than_history_is_no_window():
    c = gi.decode_ex_case(2, 2, 4, 1, 16, 20, [20, 9], "f32", seed=24)
    assert np.array_equal(orc.decode_ex(c.q, c.k, c.v, c.seqlens, c.scale, window=20),
                          orc.decode_ex(c.q, c.k, c.v, c.seqlens, c.scale))


def test_window_one_returns_own_value_row():
    c = gi.decode_ex_case(2, 3, 4, 2, 16, 20, [20, 6], "f32", seed=25)
    got = orc.decode_ex(c.q, c.k, c.v, c.seqlens, c.scale, window=1)
    for b in range(2):
        for t in range(3):
            pos = int(c.seqlens[b]) - 3 + t
            for h in range(4):
                assert np.array_equal(got[b, t, h], widen(c.v[b, pos, h // 2]))


@pytest.mark.parametrize("kv", ["same", "fp8", "e5m2"])
def test_paged_equals_contiguous(kv):
    args = dict(B=3, T=2, Hq=8, Hkv=2, d=16, Lmax=64, seqlens=[64, 33, 2], dtype="bf16", seed=26,
                kv=kv, block_size=16, window=0)
    flat = gi.decode_ex_case(**args)
    paged = gi.decode_ex_case(**args, paged=True)
    fmt = flat.kv_format or "e4m3"
    a = orc.decode_ex(flat.q, flat.k, flat.v, flat.seqlens, flat.scale, k_scale=flat.k_scale,
                      v_scale=flat.v_scale, kv_format=fmt)
    b = orc.decode_ex(paged.q, paged.k, paged.v, paged.seqlens, paged.scale, k_scale=paged.k_scale,
                      v_scale=paged.v_scale, block_table=paged.block_table,
                      block_size=paged.block_size, kv_format=fmt)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kv", ["fp8", "e5m2"])
def test_fp8_with_power_of_two_scales_equals_fp32_rows(kv):
    c = gi.decode_ex_case(2, 2, 8, 2, 32, 24, [24, 10], "f32", seed=27, kv=kv)
    ks = np.array([0.25, 2.0], np.float32)
    vs = np.array([0.5, 0.125], np.float32)
    got = orc.decode_ex(c.q, c.k, c.v, c.seqlens, c.scale, k_scale=ks, v_scale=vs,
                        kv_format=c.kv_format)
    k32 = _fp8_widen(c.k, ks, c.kv_format).astype(np.float32)   # exact: short significands times 2^k
    v32 = _fp8_widen(c.v, vs, c.kv_format).astype(np.float32)
    ref = orc.decode_ex(c.q, k32, v32, c.seqlens, c.scale)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("kv,paged,window", [("same", False, 0), ("same", True, 5),
                                             ("fp8", False, 4), ("fp8", True, 0),
                                             ("e5m2", False, 3), ("e5m2", True, 0)])
def test_matches_brute_force(kv, paged, window):
    c = gi.decode_ex_case(2, 3, 4, 2, 8, 12, [12, 5], "bf16", seed=28, kv=kv, paged=paged,
                          block_size=4, window=window)
    got = orc.decode_ex(c.q, c.k, c.v, c.seqlens, c.scale, k_scale=c.k_scale, v_scale=c.v_scale,
                        block_table=c.block_table, block_size=c.block_size, window=window,
                        kv_format=c.kv_format or "e4m3")
    if kv != "same":
        kw, vw = _fp8_widen(c.k, c.k_scale, c.kv_format), _fp8_widen(c.v, c.v_scale, c.kv_format)
    else:
        kw, vw = widen(c.k), widen(c.v)
    ref = brute.decode_ex(widen(c.q).tolist(), kw.tolist(), vw.tolist(), c.seqlens.tolist(),
                          c.scale, window=window,
                          block_table=None if c.block_table is None else c.block_table.tolist(),
                          block_size=c.block_size)
    assert np.allclose(got, np.array(ref), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kv,paged", [("same", False), ("same", True), ("fp8", True),
                                      ("e5m2", False)])
def test_append_stores_rows_exactly(kv, paged):
    c = gi.decode_ex_case(3, 4, 8, 2, 16, 32, [32, 9, 4], "bf16", seed=29, kv=kv, paged=paged,
                          block_size=8)
    k, v = c.k_pre.copy(), c.v_pre.copy()
    orc.append(k, v, c.k_new, c.v_new, c.seqlens, block_table=c.block_table,
               block_size=c.block_size)
    assert np.array_equal(k.view(np.uint8), c.k.view(np.uint8))
    assert np.array_equal(v.view(np.uint8), c.v.view(np.uint8))


def test_unappended_rows_poison_the_result():
    """The pre-append cache holds NaN where the new rows go: attending to it
    without the append must give NaN, so the append tests above are not
    vacuous."""
    c = gi.decode_ex_case(1, 2, 4, 2, 8, 10, [10], "f32", seed=30)
    assert np.isnan(orc.decode_ex(c.q, c.k_pre, c.v_pre, c.seqlens, c.scale)).all()
