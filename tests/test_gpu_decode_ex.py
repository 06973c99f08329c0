"""GPU parity of gqa_decode_ex against the fp64 CPU oracle (needs an MI355X).

Covers several new tokens per sequence, the append of their K/V rows, FP8
(E4M3 and E5M2) caches with per-KV-head scales, paged caches and sliding windows, alone
and combined, with forced and automatic splits.  Tolerance (bf16 q and out,
fp32 accumulation): |gpu - oracle| <= 2e-2 + 1e-2 |oracle| elementwise, and
every element inside the bound derived from the kernel's arithmetic
(tests/bounds.py).
Cache rows past each length, pool blocks no sequence uses and the rows of the
new tokens before the append hold NaN, so a stray read would show.
"""
import numpy as np
import pytest
import torch

import gqa_inputs as gi
import gqa_kv_cache_amd as gqa
from oracle import reference as orc
from tests import bounds as bd
from tests.gpu_util import from_dev, to_dev
from tests.helpers import bf16_tol_ok

pytestmark = pytest.mark.gpu


def _dev_cache(a):
    if a.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return to_dev(a)


def run_ex(c, append=True, num_splits=0):
    """Run gqa_decode_ex on case c; returns (out, k_cache, v_cache) on the device."""
    q = to_dev(c.q)
    k = _dev_cache(c.k_pre if append else c.k)
    v = _dev_cache(c.v_pre if append else c.v)
    sl = torch.from_numpy(c.seqlens).cuda()
    kw = {}
    if c.kv_format:
        kw["k_scale"] = torch.from_numpy(c.k_scale).cuda()
        kw["v_scale"] = torch.from_numpy(c.v_scale).cuda()
        kw["kv_format"] = c.kv_format
    if c.block_table is not None:
        kw["block_table"] = torch.from_numpy(c.block_table).cuda()
        kw["block_size"] = c.block_size
    if append:
        kw["k_new"] = _dev_cache(c.k_new)
        kw["v_new"] = _dev_cache(c.v_new)
    out = gqa.decode_ex(q, k, v, sl, scale=c.scale, window=c.window, num_splits=num_splits, **kw)
    torch.cuda.synchronize()
    return out, k, v


def oracle_ex(c, rows=None):
    return orc.decode_ex(c.q, c.k, c.v, c.seqlens, c.scale, k_scale=c.k_scale, v_scale=c.v_scale,
                         block_table=c.block_table, block_size=c.block_size, window=c.window,
                         rows=rows, kv_format=c.kv_format or "e4m3")


def check(c, got, ref):
    ok, err = bf16_tol_ok(got, ref)
    assert ok, "%s: max abs err %.3g" % (c.name, err)
    assert np.all(np.isfinite(got))
    return err


def check_oracle(c, got, rows=None):
    """Stated tolerance and derived bound against the oracle (all rows, or
    the flat ((b*T + t)*Hq + h) rows given)."""
    ref, sig, mu, kap, n = bd.ex_terms(c, rows)
    err = check(c, got, ref)
    bd.assert_within(got, ref, bd.decode_bound(ref, sig, mu, kap, n, c.q.shape[-1]), c.name)
    return err


def case(B=3, T=2, Hq=16, Hkv=4, d=128, Lmax=256, seqlens=(256, 97, 5), kv="same", paged=False,
         block_size=64, window=0, seed=40):
    name = "ex_B%d_T%d_Hq%d_Hkv%d_d%d_L%d_%s%s_w%d" % (B, T, Hq, Hkv, d, Lmax, kv,
                                                    "_paged%d" % block_size if paged else "", window)
    return gi.decode_ex_case(B, T, Hq, Hkv, d, Lmax, list(seqlens), "bf16", seed=seed, kv=kv,
                             paged=paged, block_size=block_size, window=window, name=name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T,Hq,Hkv", [(1, 8, 8), (1, 32, 4), (2, 16, 4), (4, 32, 4), (8, 64, 8),
                                      (3, 24, 2), (16, 8, 2), (64, 4, 4)])
def test_tokens_and_groups(d, T, Hq, Hkv):
    c = case(T=T, Hq=Hq, Hkv=Hkv, d=d, seqlens=(256, 97, max(T, 5)), seed=41)
    out, _, _ = run_ex(c)
    check_oracle(c, from_dev(out))


@pytest.mark.parametrize("kv", ["same", "fp8", "e5m2"])
@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7])
def test_splits(kv, splits):
    c = case(kv=kv, T=3, seqlens=(256, 200, 33), seed=42)
    out, _, _ = run_ex(c, num_splits=splits)
    check_oracle(c, from_dev(out))


@pytest.mark.parametrize("kv", ["fp8", "e5m2"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_fp8_cache(kv, d, T):
    c = case(kv=kv, d=d, T=T, Hq=32 if T == 8 else 16, seqlens=(256, 97, max(T, 5)), seed=43)
    out, _, _ = run_ex(c)
    check_oracle(c, from_dev(out))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_every_finite_code_converts_exactly(fmt):
    """One visible key: every query head returns its V row, v_scale 1.  The V
    row holds every finite code of the format (subnormals and the extremes
    included), and each is a bf16 value, so the output must equal it bit for
    bit."""
    kind = "fp8" if fmt == "e4m3" else "e5m2"
    c = case(B=1, T=1, Hq=8, Hkv=2, d=128, Lmax=32, seqlens=(1,), kv=kind, seed=52)
    val = orc.e4m3_value if fmt == "e4m3" else orc.e5m2_value
    finite = [x for x in range(256) if np.isfinite(val(x))]
    codes = np.zeros(256, np.uint8)
    codes[:len(finite)] = finite
    c.v[0, 0] = codes.reshape(2, 128)
    c.v_scale = np.ones(2, np.float32)
    out, _, _ = run_ex(c, append=False)
    want = np.array([val(int(x)) for x in codes]).reshape(2, 128)
    got = from_dev(out)[0, 0]
    for h in range(8):
        assert np.array_equal(got[h], want[h // 4]), h
    assert np.array_equal(got, oracle_ex(c)[0, 0])


def test_fp8_dtypes_name_their_format():
    """A float8_e5m2 (or float8_e4m3fn) cache needs no kv_format; a uint8 one
    is read as the kv_format it is given."""
    c = case(kv="e5m2", T=2, seed=53)
    sl = torch.from_numpy(c.seqlens).cuda()
    ks, vs = torch.from_numpy(c.k_scale).cuda(), torch.from_numpy(c.v_scale).cuda()
    k = _dev_cache(c.k).view(torch.float8_e5m2)
    v = _dev_cache(c.v).view(torch.float8_e5m2)
    out = gqa.decode_ex(to_dev(c.q), k, v, sl, scale=c.scale, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    check_oracle(c, from_dev(out))
    with pytest.raises(TypeError):
        gqa.decode_ex(to_dev(c.q), k, v, sl, scale=c.scale, k_scale=ks, v_scale=vs,
                      kv_format="e4m3")
    # the same bytes read as E4M3 are other numbers
    as_e4m3 = gqa.decode_ex(to_dev(c.q), k.view(torch.uint8), v.view(torch.uint8), sl,
                            scale=c.scale, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert not np.array_equal(from_dev(as_e4m3), from_dev(out))


@pytest.mark.parametrize("kv", ["same", "fp8", "e5m2"])
@pytest.mark.parametrize("block_size", [16, 32, 48, 64, 128])
@pytest.mark.parametrize("splits", [0, 3])
def test_paged(kv, block_size, splits):
    Lmax = -(-256 // block_size) * block_size   # whole blocks (288 for 48-row blocks)
    c = case(kv=kv, paged=True, block_size=block_size, T=2, Lmax=Lmax, seed=44)
    out, _, _ = run_ex(c, num_splits=splits)
    check_oracle(c, from_dev(out))


@pytest.mark.parametrize("window", [1, 5, 31, 32, 33, 100, 255, 4096])
@pytest.mark.parametrize("splits", [0, 4])
def test_window(window, splits):
    c = case(window=window, T=3, seqlens=(256, 130, 7), seed=45)
    out, _, _ = run_ex(c, num_splits=splits)
    check_oracle(c, from_dev(out))


@pytest.mark.parametrize("kv,block_size", [("fp8", 32), ("e5m2", 32), ("same", 16), ("fp8", 16)])
def test_everything_together(kv, block_size):
    c = case(B=4, T=4, Hq=32, Hkv=4, kv=kv, paged=True, block_size=block_size, window=45,
             seqlens=(256, 161, 64, 4), seed=46)
    for splits in (0, 1, 5):
        out, _, _ = run_ex(c, num_splits=splits)
        check_oracle(c, from_dev(out))


@pytest.mark.parametrize("kv,paged,block_size", [("same", False, 64), ("same", True, 64),
                                                 ("fp8", False, 64), ("fp8", True, 64),
                                                 ("e5m2", False, 64), ("e5m2", True, 64),
                                                 ("same", True, 16), ("fp8", True, 16)])
def test_append_writes_cache_rows_exactly(kv, paged, block_size):
    c = case(kv=kv, paged=paged, block_size=block_size, T=4, seed=47)
    out, k, v = run_ex(c, append=True)
    want_k, want_v = c.k_pre.copy(), c.v_pre.copy()
    orc.append(want_k, want_v, c.k_new, c.v_new, c.seqlens, block_table=c.block_table,
               block_size=c.block_size)
    got_k = k.view(torch.uint8).cpu().numpy().reshape(-1)
    got_v = v.view(torch.uint8).cpu().numpy().reshape(-1)
    assert np.array_equal(got_k, want_k.view(np.uint8).reshape(-1))
    assert np.array_equal(got_v, want_v.view(np.uint8).reshape(-1))
    check_oracle(c, from_dev(out))


@pytest.mark.parametrize("kv,paged,block_size", [("same", False, 64), ("fp8", True, 16),
                                                 ("e5m2", True, 32), ("same", True, 48)])
def test_append_rows_across_piece_boundaries(kv, paged, block_size):
    """The new rows straddle piece and 32-key step boundaries (rows 62-65 and
    126-129 with pieces of 32 or 64 keys): each piece stores and reads its own
    share of them, in the one launch."""
    Lmax = -(-256 // block_size) * block_size
    c = case(B=3, T=4, Hq=16, Hkv=4, kv=kv, paged=paged, block_size=block_size, Lmax=Lmax,
             seqlens=(66, 130, 4), seed=56)
    for splits in (-(-Lmax // 64), -(-Lmax // 32)):
        out, k, v = run_ex(c, append=True, num_splits=splits)
        want_k, want_v = c.k_pre.copy(), c.v_pre.copy()
        orc.append(want_k, want_v, c.k_new, c.v_new, c.seqlens, block_table=c.block_table,
                   block_size=c.block_size)
        assert np.array_equal(k.view(torch.uint8).cpu().numpy().reshape(-1), want_k.view(np.uint8).reshape(-1))
        assert np.array_equal(v.view(torch.uint8).cpu().numpy().reshape(-1), want_v.view(np.uint8).reshape(-1))
        check_oracle(c, from_dev(out))


@pytest.mark.parametrize("kv,paged,window", [("same", False, 0), ("fp8", True, 0), ("same", True, 20),
                                             ("e5m2", False, 20)])
def test_many_short_sequences_with_append(kv, paged, window):
    """256 sequences of 2-50 rows, two new tokens each stored in the same
    launch: small workgroups, pages of 16 rows, short windows."""
    lens = np.random.default_rng(57).integers(2, 51, 256)
    lens[:2] = (2, 50)
    c = case(B=256, T=2, Hq=16, Hkv=4, Lmax=64, seqlens=lens, kv=kv, paged=paged, block_size=16,
             window=window, seed=58)
    out, k, v = run_ex(c, append=True)
    want_k, want_v = c.k_pre.copy(), c.v_pre.copy()
    orc.append(want_k, want_v, c.k_new, c.v_new, c.seqlens, block_table=c.block_table,
               block_size=c.block_size)
    assert np.array_equal(k.view(torch.uint8).cpu().numpy().reshape(-1), want_k.view(np.uint8).reshape(-1))
    assert np.array_equal(v.view(torch.uint8).cpu().numpy().reshape(-1), want_v.view(np.uint8).reshape(-1))
    check_oracle(c, from_dev(out))


def _ex_fuzz_cases(n=24, seed=65):
    rng = np.random.default_rng(seed)
    for i in range(n):
        T = int(rng.choice([1, 1, 2, 3, 4, 8]))
        Hkv = int(rng.integers(1, 4))
        G = int(rng.integers(1, 64 // T + 1))                 # T * G rows per KV head, at most 64
        d = int(rng.choice([64, 128]))
        kv = str(rng.choice(["same", "same", "fp8", "e5m2"]))
        paged = bool(rng.integers(0, 2))
        bs = int(rng.choice([16, 32, 48, 64]))
        Lmax = -(-int(rng.integers(T, 700)) // bs) * bs if paged else int(rng.integers(T, 700))
        B = int(rng.integers(1, 6))
        lens = rng.integers(T, Lmax + 1, B)
        lens[0] = Lmax
        window = int(rng.choice([0, 0, 1, 17, 64, 300]))
        splits = int(rng.choice([0, 0, 1, 2, 5]))
        yield i, T, G, Hkv, d, kv, paged, bs, Lmax, tuple(int(x) for x in lens), window, min(splits, Lmax)


@pytest.mark.parametrize("i,T,G,Hkv,d,kv,paged,bs,Lmax,lens,window,splits", list(_ex_fuzz_cases()))
def test_fuzz_ex(i, T, G, Hkv, d, kv, paged, bs, Lmax, lens, window, splits):
    c = case(B=len(lens), T=T, Hq=G * Hkv, Hkv=Hkv, d=d, Lmax=Lmax, seqlens=lens, kv=kv, paged=paged,
             block_size=bs, window=window, seed=300 + i)
    out, k, v = run_ex(c, append=True, num_splits=splits)
    want_k, want_v = c.k_pre.copy(), c.v_pre.copy()
    orc.append(want_k, want_v, c.k_new, c.v_new, c.seqlens, block_table=c.block_table,
               block_size=c.block_size)
    assert np.array_equal(k.view(torch.uint8).cpu().numpy().reshape(-1), want_k.view(np.uint8).reshape(-1))
    assert np.array_equal(v.view(torch.uint8).cpu().numpy().reshape(-1), want_v.view(np.uint8).reshape(-1))
    check_oracle(c, from_dev(out))


def test_without_append_reads_the_cache():
    c = case(T=2, seed=48)
    out, _, _ = run_ex(c, append=False)
    check_oracle(c, from_dev(out))


def test_single_token_matches_plain_decode():
    c = case(T=1, Hq=64, Hkv=8, seqlens=(256, 255, 1), seed=49)
    out, k, v = run_ex(c, append=False)
    plain = gqa.decode(to_dev(np.ascontiguousarray(c.q[:, 0])), k, v,
                       torch.from_numpy(c.seqlens).cuda(), c.scale)
    torch.cuda.synchronize()
    ok, err = bf16_tol_ok(from_dev(out)[:, 0], from_dev(plain))
    assert ok, err


@pytest.mark.parametrize("kv", ["fp8", "e5m2"])
def test_fp8_70b_layer_every_row(kv):
    """The 70B-class layer shape with an FP8 cache and 4 new tokens per sequence,
    every row against the oracle."""
    c = gi.decode_ex_case(32, 4, 64, 8, 128, 4096, [4096] * 32, "bf16", seed=50, kv=kv,
                          invalid="zero", name="ex_%s_B32_T4_Hq64_Hkv8_d128_L4096" % kv)
    out, _, _ = run_ex(c)
    check_oracle(c, from_dev(out))


def test_run_twice_bitwise():
    c = case(kv="fp8", paged=True, T=3, window=50, seed=51)
    a, _, _ = run_ex(c, num_splits=3)
    b, _, _ = run_ex(c, num_splits=3)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("kv", ["same", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
def test_paged16_halves_in_different_blocks(kv, d):
    """16-row blocks: the two halves of every 32-key step come from blocks
    the random permutation put far apart; lengths end inside either half."""
    c = case(B=4, T=2, Hq=16, Hkv=2, d=d, Lmax=192, seqlens=(192, 177, 161, 2), kv=kv,
             paged=True, block_size=16, seed=54)
    for splits in (0, 1, 3):
        out, _, _ = run_ex(c, num_splits=splits)
        check_oracle(c, from_dev(out))


def test_paged16_70b_layer_every_row():
    """The 70B-class layer shape in a pool of 16-row blocks, 4 new tokens,
    every row against the oracle."""
    c = gi.decode_ex_case(32, 4, 64, 8, 128, 4096, [4096 - 7 * i for i in range(32)], "bf16",
                          seed=55, paged=True, block_size=16, invalid="zero",
                          name="ex_paged16_B32_T4_Hq64_Hkv8_d128_L4096")
    out, _, _ = run_ex(c)
    check_oracle(c, from_dev(out))


# The extended workloads the benchmark times (70B-class layer shape, seed 60,
# zero beyond each length), in the same launch configuration (automatic
# splits), every row.
L70 = dict(B=32, T=1, Hq=64, Hkv=8, d=128, Lmax=4096, seqlens=[4096] * 32, dtype="bf16",
           invalid="zero")


@pytest.mark.parametrize("name,extra", [
    ("decode_ex_e4m3_B32_Hq64_Hkv8_d128_L4096", dict(kv="fp8")),
    ("decode_ex_e5m2_B32_Hq64_Hkv8_d128_L4096", dict(kv="e5m2")),
    ("decode_ex_bf16_T4_B32_Hq64_Hkv8_d128_L4096", dict(T=4)),
    ("decode_ex_bf16_paged64_B32_Hq64_Hkv8_d128_L4096", dict(paged=True, block_size=64)),
    ("decode_ex_bf16_paged16_B32_Hq64_Hkv8_d128_L4096", dict(paged=True, block_size=16)),
    ("decode_ex_bf16_window1024_B32_Hq64_Hkv8_d128_L4096", dict(window=1024)),
])
def test_benchmark_extended_workloads_every_row(name, extra):
    a = dict(L70)
    a.update(extra)
    c = gi.decode_ex_case(seed=60, name=name, **a)
    out, _, _ = run_ex(c, append=False)
    check_oracle(c, from_dev(out))
