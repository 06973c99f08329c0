"""GPU parity of gqa_decode against the fp64 CPU oracle (needs an MI355X).

Tolerances: fp32 inputs max |gpu - oracle| <= 1e-5; bf16 inputs (fp32
accumulation) |gpu - oracle| <= 2e-2 + 1e-2 |oracle| elementwise.  Beside
them every element must lie inside the bound derived from the kernel's
arithmetic (tests/bounds.py), tens of times tighter at long lengths.  Cache
rows at or beyond seqlens[b] hold NaN, so any read of them would show.
"""
import numpy as np
import pytest
import torch

import gqa_inputs as gi
import gqa_kv_cache_amd as gqa
from oracle import reference as orc
from tests import bounds as bd
from tests.gpu_util import bits, from_dev, to_dev
from tests.helpers import bf16_tol_ok, f32_tol_ok, widen

pytestmark = pytest.mark.gpu


def run_decode(case, num_splits=0, out=None, workspace=None):
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    sl = torch.from_numpy(case.seqlens).cuda()
    o = gqa.decode(q, k, v, sl, case.scale, out=out, num_splits=num_splits, workspace=workspace)
    torch.cuda.synchronize()
    return o


def check(case, got, ref):
    if case.dtype == "f32":
        ok, err = f32_tol_ok(got, ref)
    else:
        ok, err = bf16_tol_ok(got, ref)
    assert ok, "%s: max abs err %.3g" % (case.name, err)
    assert np.all(np.isfinite(got))
    return err


def check_oracle(case, got, rows=None):
    """Stated tolerance and derived bound against the oracle (all rows, or
    the flat b*Hq + h rows given; got holds exactly those rows)."""
    ref, sig, mu, kap, n = bd.decode_terms(case, rows)
    err = check(case, got, ref)
    d = case.q.shape[-1]
    bound = (bd.decode_bound_f32 if case.dtype == "f32" else bd.decode_bound)(ref, sig, mu, kap, n, d)
    bd.assert_within(got, ref, bound, case.name)
    return err


# --- the tiny fp32 workload: GQA, MHA and MQA on the same q ---------------

@pytest.mark.parametrize("hkv", [2, 8, 1])
@pytest.mark.parametrize("splits", [0, 1, 2, 3, 5])
def test_tiny_fp32(hkv, splits):
    c = gi.tiny_decode(hkv)
    check_oracle(c, from_dev(run_decode(c, splits)))


# --- the 70B-class layer: full output against the oracle ------------------

def test_decode_70b_full():
    c = gi.decode_70b()
    err = check_oracle(c, from_dev(run_decode(c)))
    print("decode 70b max abs err %.3g" % err)


@pytest.mark.parametrize("splits", [1, 2, 8])
def test_decode_70b_forced_splits_full(splits):
    c = gi.decode_70b()
    check_oracle(c, from_dev(run_decode(c, splits)))


# --- head-sharing sweep ----------------------------------------------------

@pytest.mark.parametrize("hkv", gi.SWEEP_HKV)
def test_sweep_full(hkv):
    c = gi.sweep_decode(hkv)
    check_oracle(c, from_dev(run_decode(c)))


# --- ragged batch at full size, NaN beyond every length, every row ----------

def test_ragged_full():
    c = gi.ragged_decode(invalid="nan")
    got = from_dev(run_decode(c))
    assert np.all(np.isfinite(got))
    check_oracle(c, got)


# --- many short sequences: one small workgroup each, some with no rows ------

@pytest.mark.parametrize("dtype,B,Hq,Hkv,d", [("bf16", 1024, 32, 8, 128), ("f32", 512, 8, 2, 64)])
@pytest.mark.parametrize("splits", [0, 2, 3])
def test_many_short_sequences(dtype, B, Hq, Hkv, d, splits):
    lens = np.random.default_rng(61).integers(0, 41, B).astype(np.int32)
    lens[:3] = (0, 40, 1)
    c = gi.decode_case(B, Hq, Hkv, d, 40, lens, dtype, q_seed=62, kv_seed=63, invalid="nan",
                       name="many_short_%s" % dtype)
    got = from_dev(run_decode(c, splits))
    check_oracle(c, got)
    assert not np.any(got.reshape(B, -1)[lens == 0])   # no visible row: zero output


# --- seeded fuzz over group size, head dim, dtype, lengths and pieces -------

def _fuzz_cases(n=32, seed=64):
    rng = np.random.default_rng(seed)
    for i in range(n):
        dtype = "f32" if i % 4 == 3 else "bf16"
        G = int(rng.integers(1, 65))
        Hkv = int(rng.integers(1, 4))
        d = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 7))
        Lmax = int(rng.integers(1, 1201))
        lens = rng.integers(0, Lmax + 1, B).astype(np.int32)
        lens[0] = Lmax
        splits = int(rng.choice([0, 0, 1, 2, 3, 5, 9]))
        yield i, dtype, G, Hkv, d, Lmax, tuple(int(x) for x in lens), min(splits, Lmax)


@pytest.mark.parametrize("i,dtype,G,Hkv,d,Lmax,lens,splits", list(_fuzz_cases()))
def test_fuzz(i, dtype, G, Hkv, d, Lmax, lens, splits):
    c = gi.decode_case(len(lens), G * Hkv, Hkv, d, Lmax, list(lens), dtype, q_seed=100 + i,
                       kv_seed=200 + i, invalid="nan", name="fuzz%d" % i)
    check_oracle(c, from_dev(run_decode(c, splits)))


# --- randomised shapes: head dims, group sizes, lengths, ragged, splits ------

SEQ = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 300]


def _sweep_cases():
    for d in (64, 128):
        for G in (1, 2, 4, 8, 16, 64):
            Hkv = 2 if G <= 16 else 1
            for splits in (1, 3, 0):
                yield ("bf16", d, G * Hkv, Hkv, splits)
    for d in (64, 128):
        for G in (1, 4, 16, 64):
            for splits in (1, 4):
                yield ("f32", d, G, 1, splits)


@pytest.mark.parametrize("dtype,d,Hq,Hkv,splits", list(_sweep_cases()))
def test_shapes_ragged_nan_poisoned(dtype, d, Hq, Hkv, splits):
    c = gi.decode_case(len(SEQ), Hq, Hkv, d, 300, SEQ, dtype, q_seed=d + Hq, kv_seed=Hkv + splits,
                       invalid="nan", name="sweep_%s_d%d_Hq%d_Hkv%d_s%d" % (dtype, d, Hq, Hkv, splits))
    got = from_dev(run_decode(c, splits))
    check_oracle(c, got)
    assert np.all(got[0] == 0.0)  # zero-length sequence


@pytest.mark.parametrize("G,Hkv", [(49, 1), (56, 2), (63, 1)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_partial_last_head_tile(G, Hkv, d, splits):
    """Groups of 49..63 heads: four 16-head tiles, the last one partly empty."""
    c = gi.decode_case(len(SEQ), G * Hkv, Hkv, d, 300, SEQ, "bf16", q_seed=G + d, kv_seed=G + splits,
                       invalid="nan", name="partial_tile_G%d_Hkv%d_d%d_s%d" % (G, Hkv, d, splits))
    got = from_dev(run_decode(c, splits))
    check_oracle(c, got)
    assert np.all(got[0] == 0.0)  # zero-length sequence


@pytest.mark.parametrize("splits", [1, 2, 7, 0])
def test_long_two_sequences(splits):
    c = gi.decode_case(2, 16, 2, 128, 4096, [4096, 4000], "bf16", q_seed=5, kv_seed=6, invalid="nan")
    check_oracle(c, from_dev(run_decode(c, splits)))


@pytest.mark.parametrize("B,Hq,Hkv,L,lens,splits", [
    (32, 64, 1, 4096, None, 0),                  # automatic: 8 pieces of 512 keys
    (3, 57, 1, 1100, [1100, 700, 513], 2),       # partly empty last head tile, 550-key pieces
    (2, 128, 2, 1536, [1536, 1000], 1),          # one 1536-key piece
])
def test_four_head_tiles_long_pieces(B, Hq, Hkv, L, lens, splits):
    """Groups of 49-64 heads with pieces of 512 keys or more (the waves split
    the keys and combine four tiles of partial sums)."""
    lens = lens or [L] * B
    c = gi.decode_case(B, Hq, Hkv, 128, L, lens, "bf16", q_seed=13, kv_seed=14, invalid="nan",
                       name="tiles4_long_B%d_Hq%d_Hkv%d_L%d_s%d" % (B, Hq, Hkv, L, splits))
    check_oracle(c, from_dev(run_decode(c, splits)))


@pytest.mark.timeout(400)  # 2.1 GB of cache to draw and an fp64 oracle over half a million keys
def test_longest_cache_the_offsets_allow():
    """Lmax = 524,255 is the largest length the 32-bit offset check admits at
    Hkv 8, d 128 ((Lmax + 32) * Hkv * d * 4 <= 2^31 - 1); one more is refused.
    The automatic plan cuts it into 64 pieces of 8,192 keys."""
    Lmax = 524255
    with pytest.raises(gqa.GqaError):
        gqa.decode_workspace_size(1, 64, 8, 128, Lmax + 1, gqa.BF16, 0)
    assert gqa.decode_num_splits(1, 64, 8, 128, Lmax, gqa.BF16, 0) == 64
    c = gi.decode_case(1, 64, 8, 128, Lmax, [Lmax], "bf16", q_seed=17, kv_seed=18, invalid="nan",
                       name="decode_longest_B1_Hq64_Hkv8_d128_L524255")
    check_oracle(c, from_dev(run_decode(c)))


def test_one_key_per_split():
    c = gi.decode_case(3, 8, 2, 128, 100, [100, 57, 1], "bf16", q_seed=7, kv_seed=8, invalid="nan")
    check_oracle(c, from_dev(run_decode(c, 100)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_key_returns_v_exactly(dtype):
    c = gi.decode_case(4, 16, 4, 128, 8, [1, 1, 1, 1], dtype, q_seed=9, kv_seed=10, invalid="nan")
    got = from_dev(run_decode(c, 1))
    for b in range(4):
        for h in range(16):
            assert np.array_equal(got[b, h], widen(c.v[b, 0, h // 4]))


def test_gqa_equals_repeat_expanded_mha_on_gpu():
    c = gi.decode_case(3, 32, 4, 128, 500, [500, 321, 77], "bf16", q_seed=11, kv_seed=12, invalid="nan")
    gs = 8
    m = gi.DecodeCase("mha", c.q, np.ascontiguousarray(np.repeat(c.k, gs, axis=2)),
                      np.ascontiguousarray(np.repeat(c.v, gs, axis=2)), c.seqlens, c.scale, "bf16")
    a = from_dev(run_decode(c))
    b = from_dev(run_decode(m))
    ok, err = bf16_tol_ok(a, b)
    assert ok, err


# --- memory safety and determinism ------------------------------------------

def test_guard_bands_untouched():
    c = gi.decode_case(4, 32, 8, 128, 1000, [1000, 999, 3, 640], "bf16", q_seed=13, kv_seed=14,
                       invalid="nan")
    splits = 4
    n_out = 4 * 32 * 128
    guard = 4096
    canary = 0x5A5A
    out_big = torch.full((n_out + 2 * guard,), canary, dtype=torch.int16, device="cuda")
    out = out_big[guard:guard + n_out].view(torch.bfloat16).view(4, 32, 128)
    need = gqa.decode_workspace_size(4, 32, 8, 128, 1000, gqa.BF16, splits)
    assert need > 0
    ws_big = torch.full((need + 2 * guard,), 0x77, dtype=torch.uint8, device="cuda")
    ws = ws_big[guard:guard + need]
    run_decode(c, splits, out=out, workspace=ws)
    ob = out_big.cpu().numpy()
    assert np.all(ob[:guard] == canary) and np.all(ob[guard + n_out:] == canary)
    wb = ws_big.cpu().numpy()
    assert np.all(wb[:guard] == 0x77) and np.all(wb[guard + need:] == 0x77)
    check_oracle(c, from_dev(out))


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_run_twice_bitwise(splits):
    c = gi.decode_case(8, 64, 8, 128, 2048, [2048, 1, 700, 2047, 33, 1024, 5, 1500], "bf16",
                       q_seed=15, kv_seed=16, invalid="nan")
    a = bits(run_decode(c, splits))
    b = bits(run_decode(c, splits))
    assert np.array_equal(a, b)


def test_concurrent_threads_and_streams_bitwise():
    """Two host threads, each on its own stream (default priority), issue
    decode and extended-decode calls back to back; every output equals the
    single-stream result bit for bit (the calls keep no shared state)."""
    import threading
    c1 = gi.decode_case(4, 32, 8, 128, 1000, [1000, 999, 3, 640], "bf16", q_seed=21, kv_seed=22,
                        invalid="nan")
    c2 = gi.decode_ex_case(3, 2, 16, 4, 128, 256, [256, 97, 5], "bf16", seed=23, kv="fp8",
                           paged=True, block_size=16, window=50)
    want1 = bits(run_decode(c1, 3))

    def ex_args():
        d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda() if a.dtype == np.uint8 else to_dev(a)
        return (to_dev(c2.q), d(c2.k), d(c2.v), torch.from_numpy(c2.seqlens).cuda(),
                dict(scale=c2.scale, k_scale=torch.from_numpy(c2.k_scale).cuda(),
                     v_scale=torch.from_numpy(c2.v_scale).cuda(),
                     block_table=torch.from_numpy(c2.block_table).cuda(), block_size=16, window=50))

    q2, k2, v2, sl2, kw2 = ex_args()
    want2 = bits(gqa.decode_ex(q2, k2, v2, sl2, num_splits=2, **kw2))
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(name):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                if name == "decode":
                    q, k, v = to_dev(c1.q), to_dev(c1.k), to_dev(c1.v)
                    sl = torch.from_numpy(c1.seqlens).cuda()
                    outs = [gqa.decode(q, k, v, sl, c1.scale, num_splits=3) for _ in range(20)]
                else:
                    q, k, v, sl, kw = ex_args()
                    outs = [gqa.decode_ex(q, k, v, sl, num_splits=2, **kw) for _ in range(20)]
            s.synchronize()
            results[name] = [bits(o) for o in outs]
        except Exception as e:  # surfaced below, in the test's own thread
            errors.append(repr(e))

    ts = [threading.Thread(target=worker, args=(n,)) for n in ("decode", "ex")]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=60)
    assert not errors, errors
    assert all(np.array_equal(o, want1) for o in results["decode"])
    assert all(np.array_equal(o, want2) for o in results["ex"])
    ok, err = bf16_tol_ok(widen(want2.view(np.uint16)).reshape(c2.q.shape),
                          orc.decode_ex(c2.q, c2.k, c2.v, c2.seqlens, c2.scale, k_scale=c2.k_scale,
                                        v_scale=c2.v_scale, block_table=c2.block_table,
                                        block_size=16, window=50))
    assert ok, err
