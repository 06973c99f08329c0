"""GPU parity of gqa_prefill against the fp64 CPU oracle (needs an MI355X).

bf16 inputs with fp32 accumulation: |gpu - oracle| <= 2e-2 + 1e-2 |oracle|,
and, for causal prompts, every element inside the bound derived from the
kernel's arithmetic (bf16 weights shared by the weighted sum and the weight
sum; tests/bounds.py).
"""
import numpy as np
import pytest
import torch

import gqa_inputs as gi
import gqa_kv_cache_amd as gqa
from oracle import reference as orc
from tests import bounds as bd
from tests.gpu_util import bits, from_dev, to_dev
from tests.helpers import bf16_tol_ok, widen

pytestmark = pytest.mark.gpu


def run_prefill(c):
    o = gqa.prefill(to_dev(c.q), to_dev(c.k), to_dev(c.v), causal=c.causal, scale=c.scale)
    torch.cuda.synchronize()
    return o


def check(name, got, ref):
    ok, err = bf16_tol_ok(got, ref)
    assert ok, "%s: max abs err %.3g" % (name, err)
    assert np.all(np.isfinite(got))


def check_causal(name, p, got, rows=None, window=0, scale=None):
    """Stated tolerance and derived bound against the causal oracle (all rows
    or the flat (b*P + i)*Hq + h rows given), optionally with a window."""
    B, P, Hq, d = p.q.shape
    ref, sig, mu, kap = orc.decode_ex(p.q, p.k, p.v, np.full(B, P, np.int32),
                                      p.scale if scale is None else scale, window=window,
                                      rows=rows, terms=True)
    flat = np.arange(B * P * Hq) if rows is None else np.asarray(rows, np.int64)
    i = (flat // Hq) % P
    n = np.minimum(i + 1, window) if window > 0 else i + 1
    if rows is None:
        n = n.reshape(B, P, Hq)
    check(name, got, ref)
    return bd.assert_within(got, ref, bd.prefill_bound(ref, sig, mu, kap, n, d), name)


def _cases():
    for causal in (True, False):
        for (B, P, Hq, Hkv, d) in [(1, 1, 4, 1, 128), (2, 7, 8, 2, 128), (1, 64, 4, 4, 128),
                                   (1, 65, 8, 1, 128), (2, 200, 6, 3, 64), (1, 129, 16, 2, 64),
                                   (1, 300, 2, 2, 128), (1, 97, 64, 1, 128)]:
            yield causal, B, P, Hq, Hkv, d


@pytest.mark.parametrize("causal,B,P,Hq,Hkv,d", list(_cases()))
def test_small_full(causal, B, P, Hq, Hkv, d):
    c = gi.prefill_case(B, P, Hq, Hkv, d, "bf16", seed=P + Hq + d, causal=causal)
    got = from_dev(run_prefill(c))
    if causal:
        check_causal("prefill", c, got)
    else:
        check("prefill", got, orc.prefill(c.q, c.k, c.v, causal, c.scale))


def test_medium_full():
    c = gi.prefill_case(1, 1024, 16, 4, 128, "bf16", seed=77)
    check_causal("prefill_1024", c, from_dev(run_prefill(c)))


@pytest.mark.timeout(400)  # the fp64 oracle of every row takes about a minute
def test_causal_prefill_full_size_every_row():
    """The causal prefill workload (B2 P4096 Hq32 Hkv8 d128): all 262,144
    output rows against the oracle."""
    c = gi.prefill_causal()
    got = from_dev(run_prefill(c))
    r = check_causal(c.name, c, got)
    print("prefill full size: largest err / derived bound %.3f" % r)


def test_prefill_rows_match_decode_on_gpu():
    """Causal prefill row i equals decode over i+1 cached rows (both on the GPU)."""
    B, P, Hq, Hkv, d = 2, 160, 8, 2, 128
    c = gi.prefill_case(B, P, Hq, Hkv, d, "bf16", seed=88)
    pre = from_dev(run_prefill(c))
    k, v = to_dev(c.k), to_dev(c.v)
    for i in (0, 1, 31, 32, 100, 159):
        q = to_dev(np.ascontiguousarray(c.q[:, i]))
        sl = torch.full((B,), i + 1, dtype=torch.int32, device="cuda")
        dec = from_dev(gqa.decode(q, k, v, sl, c.scale))
        ok, err = bf16_tol_ok(pre[:, i], dec)
        assert ok, (i, err)


def test_prefill_run_twice_bitwise():
    c = gi.prefill_case(1, 333, 16, 4, 128, "bf16", seed=99)
    assert np.array_equal(bits(run_prefill(c)), bits(run_prefill(c)))


def test_prefill_guard_bands_untouched():
    """The kernel writes exactly the output rows: canaries around them survive."""
    B, P, Hq, Hkv, d = 2, 203, 8, 2, 128
    c = gi.prefill_case(B, P, Hq, Hkv, d, "bf16", seed=101)
    n_out = B * P * Hq * d
    guard = 4096
    canary = 0x5A5A
    out_big = torch.full((n_out + 2 * guard,), canary, dtype=torch.int16, device="cuda")
    out = out_big[guard:guard + n_out].view(torch.bfloat16).view(B, P, Hq, d)
    gqa.prefill(to_dev(c.q), to_dev(c.k), to_dev(c.v), causal=True, scale=c.scale, out=out)
    torch.cuda.synchronize()
    ob = out_big.cpu().numpy()
    assert np.all(ob[:guard] == canary) and np.all(ob[guard + n_out:] == canary)
    check_causal("prefill_guarded", c, from_dev(out))


@pytest.mark.parametrize("shape", [(1, 150, 8, 2, 128), (2, 77, 4, 4, 64)])
def test_prefill_scale_zero_is_running_mean(shape):
    """Scale 0 makes every visible key weigh the same: causal row i is the mean
    of V rows 0..i of its group (a closed form, independent of the oracle)."""
    B, P, Hq, Hkv, d = shape
    c = gi.prefill_case(B, P, Hq, Hkv, d, "bf16", seed=103)
    out = gqa.prefill(to_dev(c.q), to_dev(c.k), to_dev(c.v), causal=True, scale=0.0)
    torch.cuda.synchronize()
    got = from_dev(out)
    v = widen(c.v)                                   # [B, P, Hkv, d] exact
    mean = np.cumsum(v, axis=1) / np.arange(1, P + 1)[None, :, None, None]
    ref = np.repeat(mean, Hq // Hkv, axis=2)         # head h reads KV head h // (Hq/Hkv)
    ok, err = bf16_tol_ok(got, ref)
    assert ok, err


# --- sliding-window prefill (gqa_prefill_ex) --------------------------------
# The oracle is the extended decode with one new token per prompt position
# over the prompt's own K/V: token t sits at position t and sees the last
# `window` keys up to it.

@pytest.mark.parametrize("shape", [(2, 200, 8, 2, 128), (1, 97, 4, 4, 64), (2, 333, 16, 8, 128)])
@pytest.mark.parametrize("window", [1, 7, 32, 63, 64, 65, 100, 1000])
def test_window_prefill_small(shape, window):
    B, P, Hq, Hkv, d = shape
    p = gi.prefill_case(B, P, Hq, Hkv, d, "bf16", seed=70 + window)
    out = gqa.prefill(to_dev(p.q), to_dev(p.k), to_dev(p.v), True, p.scale, window=window)
    torch.cuda.synchronize()
    check_causal("window_%d" % window, p, from_dev(out), window=window)


@pytest.mark.parametrize("window", [0, 40])
def test_prefill_many_sequences(window):
    """Twelve prompts, groups of three heads (one head per workgroup): the
    workgroup-to-(sequence, head set, row block) mapping away from B = 1, 2."""
    p = gi.prefill_case(12, 90, 12, 4, 128, "bf16", seed=90 + window)
    out = gqa.prefill(to_dev(p.q), to_dev(p.k), to_dev(p.v), True, p.scale, window=window)
    torch.cuda.synchronize()
    check_causal("many_sequences_%d" % window, p, from_dev(out), window=window)


def _prefill_fuzz_cases(n=20, seed=66):
    rng = np.random.default_rng(seed)
    for i in range(n):
        Hkv = int(rng.integers(1, 5))
        G = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 16]))
        d = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 4))
        P = int(rng.integers(1, 400))
        window = int(rng.choice([0, 0, 0, 1, 31, 33, 100]))
        yield i, B, P, G * Hkv, Hkv, d, window


@pytest.mark.parametrize("i,B,P,Hq,Hkv,d,window", list(_prefill_fuzz_cases()))
def test_fuzz_prefill(i, B, P, Hq, Hkv, d, window):
    p = gi.prefill_case(B, P, Hq, Hkv, d, "bf16", seed=400 + i)
    out = gqa.prefill(to_dev(p.q), to_dev(p.k), to_dev(p.v), True, p.scale, window=window)
    torch.cuda.synchronize()
    check_causal("fuzz%d" % i, p, from_dev(out), window=window)


@pytest.mark.timeout(400)  # the fp64 oracle of every row takes about a minute
def test_window_prefill_full_size_every_row():
    p = gi.prefill_case(2, 4096, 32, 8, 128, "bf16", seed=5)
    out = gqa.prefill(to_dev(p.q), to_dev(p.k), to_dev(p.v), True, p.scale, window=1024)
    torch.cuda.synchronize()
    check_causal("window_1024_full_size", p, from_dev(out), window=1024)


def test_window_at_least_prompt_is_plain_causal():
    p = gi.prefill_case(1, 150, 8, 2, 128, "bf16", seed=79)
    a = gqa.prefill(to_dev(p.q), to_dev(p.k), to_dev(p.v), True, p.scale)
    b = gqa.prefill(to_dev(p.q), to_dev(p.k), to_dev(p.v), True, p.scale, window=150)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# --- references that move along the prompt ----------------------------------
# Key rows grow in magnitude along the prompt, so the running maximum of a
# row's scores keeps rising and the kernel's lazily moved reference (an
# integer, moved by an exact power-of-two rescale of O, the weight sums and
# the weights already formed) is exercised on many chunks, for both halves of
# a wave's row tiles, including a single large jump.

@pytest.mark.parametrize("profile", ["linear", "exp", "jump"])
@pytest.mark.parametrize("shape", [(1, 640, 8, 2, 128, True, 0), (2, 515, 12, 3, 64, True, 0),
                                   (1, 700, 8, 8, 128, False, 0), (1, 600, 8, 2, 128, True, 200)])
def test_prefill_moving_references(profile, shape):
    B, P, Hq, Hkv, d, causal, window = shape
    p = gi.prefill_growing_keys(B, P, Hq, Hkv, d, seed=120 + P, profile=profile, causal=causal)
    out = gqa.prefill(to_dev(p.q), to_dev(p.k), to_dev(p.v), causal, p.scale, window=window)
    torch.cuda.synchronize()
    got = from_dev(out)
    if causal:
        check_causal("moving_%s" % profile, p, got, window=window)
    else:
        check("moving_%s" % profile, got, orc.prefill(p.q, p.k, p.v, causal, p.scale))


def test_prefill_moving_references_negative_scale():
    p = gi.prefill_growing_keys(1, 300, 8, 2, 128, seed=131, profile="linear")
    out = gqa.prefill(to_dev(p.q), to_dev(p.k), to_dev(p.v), True, -p.scale)
    torch.cuda.synchronize()
    check_causal("moving_negative_scale", p, from_dev(out), scale=-p.scale)
