"""Host-side checks of the C ABI: exports, header, argument validation, counts.

No test here launches GPU work: every call either is a pure host function
(counts, planning with an explicit split count) or fails validation before
the library touches the HIP runtime.
"""
import ctypes
import os
import re
import subprocess

import pytest

import gqa_inputs as gi
import gqa_kv_cache_amd as gqa
from gqa_kv_cache_amd._native import Status
from oracle import counts as oc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")

FAKE = 0x10000  # aligned, non-null; never dereferenced by the validation paths used here


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = gqa.load()
    names = declared_functions()
    assert len(names) >= 10
    assert set(names) == set(gqa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", gqa.LIBRARY_PATH], capture_output=True,
                         text=True, check=True).stdout
    for n in names:
        assert re.search(r"\bT %s$" % n, out, flags=re.M), n


def test_header_is_plain_c99(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "gqa.h"\nint main(void){ return (int)GQA_OK; }\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-fsyntax-only",
                    "-I", os.path.dirname(HEADER), str(src)], check=True)


def _decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sl=FAKE, B=2, Hq=8, Hkv=2, d=128, Lmax=64, scale=0.1,
             dt=gqa.BF16, out=FAKE, ws=None, wsb=0, ns=1, stream=None)
    a.update(kw)
    return gqa.load().gqa_decode(a["q"], a["k"], a["v"], a["sl"], a["B"], a["Hq"], a["Hkv"], a["d"],
                                 a["Lmax"], a["scale"], a["dt"], a["out"], a["ws"], a["wsb"],
                                 a["ns"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), Status.ERR_NULL),
    (dict(sl=None), Status.ERR_NULL),
    (dict(out=None), Status.ERR_NULL),
    (dict(k=FAKE + 2), Status.ERR_ALIGN),
    (dict(out=FAKE + 8), Status.ERR_ALIGN),
    (dict(B=0), Status.ERR_SHAPE),
    (dict(Lmax=0), Status.ERR_SHAPE),
    (dict(Hkv=0), Status.ERR_SHAPE),
    (dict(Hq=6, Hkv=4), Status.ERR_GROUP),
    (dict(d=96), Status.ERR_HEADDIM),
    (dict(d=256), Status.ERR_HEADDIM),
    (dict(dt=7), Status.ERR_DTYPE),
    (dict(Hq=128, Hkv=1), Status.ERR_UNSUPPORTED),
    (dict(ns=-1), Status.ERR_UNSUPPORTED),
    (dict(ns=65), Status.ERR_UNSUPPORTED),
    (dict(ns=4, ws=None), Status.ERR_WORKSPACE),
    (dict(ns=4, ws=FAKE, wsb=16), Status.ERR_WORKSPACE),
    (dict(ns=4, ws=FAKE + 4, wsb=1 << 30), Status.ERR_WORKSPACE),
    # one sequence's cache slice is addressed with 32-bit byte offsets:
    # (Lmax + 32) * Hkv * d * 4 = 2097153 * 1024 > 2^31 - 1
    (dict(Lmax=2097121), Status.ERR_SHAPE),
])
def test_decode_validation(kw, expect):
    assert _decode(**kw) == expect


def _decode_noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sl=FAKE, B=2, Hq=8, Hkv=2, d=128, Lmax=64, scale=0.1,
             dt=gqa.BF16, out=FAKE, ns=1, stream=None)
    a.update(kw)
    return gqa.load().gqa_decode_noalloc(a["q"], a["k"], a["v"], a["sl"], a["B"], a["Hq"], a["Hkv"],
                                         a["d"], a["Lmax"], a["scale"], a["dt"], a["out"], a["ns"],
                                         a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), Status.ERR_NULL),
    (dict(out=None), Status.ERR_NULL),
    (dict(v=FAKE + 2), Status.ERR_ALIGN),
    (dict(B=0), Status.ERR_SHAPE),
    (dict(Hq=6, Hkv=4), Status.ERR_GROUP),
    (dict(d=96), Status.ERR_HEADDIM),
    (dict(dt=gqa.FP8_E4M3), Status.ERR_DTYPE),
    (dict(ns=65), Status.ERR_UNSUPPORTED),
    (dict(Lmax=2097121), Status.ERR_SHAPE),
    # partials of 2 x 8 heads x 64 pieces x (128 + 2) x 4 B = 532,480 B fit; at
    # 64 x 64 heads x 64 pieces they take 136 MB, above the 16 MiB scratch
    (dict(B=64, Hq=64, Hkv=8, ns=64), Status.ERR_SCRATCH_LIMIT),
    (dict(B=2, Hq=512, Hkv=8, Lmax=8192, ns=64), Status.ERR_SCRATCH_LIMIT),
])
def test_decode_noalloc_validation(kw, expect):
    """Every error returns before the library touches the device."""
    assert _decode_noalloc(**kw) == expect


def test_noalloc_scratch_limit_is_the_documented_size():
    text = open(HEADER).read()
    assert re.search(r"#define GQA_NOALLOC_SCRATCH_BYTES \(\(size_t\)16 << 20\)", text)
    limit = 16 << 20
    # B * Hq * pieces * (d + 2) * 4 bytes: 2 x 64 x 252 x 130 x 4 = 16,773,120 fits,
    # 253 pieces (16,839,680) do not
    assert gqa.decode_workspace_size(2, 64, 8, 128, 252, gqa.BF16, 252) == 16773120 <= limit
    assert gqa.decode_workspace_size(2, 64, 8, 128, 253, gqa.BF16, 253) == 16839680 > limit
    assert _decode_noalloc(B=2, Hq=64, Hkv=8, Lmax=253, ns=253) == Status.ERR_SCRATCH_LIMIT


def _prefill(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, P=16, Hq=8, Hkv=2, d=128, causal=1, scale=0.1,
             dt=gqa.BF16, out=FAKE, stream=None)
    a.update(kw)
    return gqa.load().gqa_prefill(a["q"], a["k"], a["v"], a["B"], a["P"], a["Hq"], a["Hkv"], a["d"],
                                  a["causal"], a["scale"], a["dt"], a["out"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(v=None), Status.ERR_NULL),
    (dict(q=FAKE + 2), Status.ERR_ALIGN),
    (dict(P=0), Status.ERR_SHAPE),
    (dict(Hq=8, Hkv=3), Status.ERR_GROUP),
    (dict(d=32), Status.ERR_HEADDIM),
    (dict(dt=gqa.F32), Status.ERR_DTYPE),
    (dict(Hq=65 * 2, Hkv=2), Status.ERR_UNSUPPORTED),
    # K/V chunk byte offsets are 32-bit: (P + 128) * Hkv * d * 2 = 2^31 > 2^31 - 1
    (dict(P=4194176), Status.ERR_SHAPE),
])
def test_prefill_validation(kw, expect):
    assert _prefill(**kw) == expect


def test_status_strings():
    for s in Status:
        assert gqa.status_str(int(s)).startswith("GQA_")
    assert "unknown" in gqa.status_str(99)


@pytest.mark.parametrize("Lmax,ns,expect", [(4096, 4, 4), (4096, 1, 1), (10, 4, 4), (10, 6, 5),
                                            (10, 10, 10), (1, 1, 1), (32768, 16, 16)])
def test_forced_split_plan(Lmax, ns, expect):
    assert gqa.decode_num_splits(4, 8, 2, 128, Lmax, gqa.BF16, ns) == expect
    ws = gqa.decode_workspace_size(4, 8, 2, 128, Lmax, gqa.BF16, ns)
    assert ws == (0 if expect == 1 else 4 * 8 * expect * (128 + 2) * 4)


# --- library counts against the oracle's independently written counts -----

def _workloads():
    yield "tiny", [128], 8, 2, 64, 4
    yield "70b", [4096] * 32, 64, 8, 128, 2
    for h in gi.SWEEP_HKV:
        yield "sweep%d" % h, [2048] * 16, 64, h, 128, 2
    yield "ragged", list(gi.ragged_seqlens()), 32, 8, 128, 2


@pytest.mark.parametrize("name,seq,Hq,Hkv,d,elt", list(_workloads()), ids=lambda x: str(x)[:12])
def test_decode_counts_match_oracle(name, seq, Hq, Hkv, d, elt):
    dt = gqa.BF16 if elt == 2 else gqa.F32
    assert gqa.decode_bytes(seq, Hq, Hkv, d, dt) == oc.decode_bytes(seq, Hq, Hkv, d, elt)
    assert gqa.decode_flops(seq, Hq, d) == oc.decode_flops(seq, Hq, d)


def test_decode_bytes_headline_value():
    # K+V = 2*32*4096*8*128*2 bytes, plus q and out once each
    assert gqa.decode_bytes([4096] * 32, 64, 8, 128, gqa.BF16) == 537919488


@pytest.mark.parametrize("L,Hkv,d", [(1, 1, 1), (4096, 8, 128), (32768, 8, 128), (131072, 32, 128)])
def test_kv_elems_match_oracle(L, Hkv, d):
    assert gqa.kv_cache_elems(L, Hkv, d) == oc.kv_cache_elems(L, Hkv, d)


@pytest.mark.parametrize("B,P,Hq,Hkv,d", [(2, 4096, 32, 8, 128), (1, 1, 4, 4, 64), (3, 77, 8, 2, 128)])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_counts_match_oracle(B, P, Hq, Hkv, d, causal):
    assert gqa.prefill_flops(B, P, Hq, d, causal) == oc.prefill_flops(B, P, Hq, d, causal)
    assert gqa.prefill_bytes(B, P, Hq, Hkv, d, gqa.BF16) == oc.prefill_bytes(B, P, Hq, Hkv, d, 2)


def test_prefill_flops_headline_value():
    assert gqa.prefill_flops(2, 4096, 32, 128, True) == 274945015808


# --- gqa_decode_ex ---------------------------------------------------------

from gqa_kv_cache_amd._native import DecodeExArgs  # noqa: E402


def _ex_args(**kw):
    a = DecodeExArgs()
    base = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, seqlens=FAKE, B=2, T=2, Hq=8, Hkv=2, d=128,
                Lmax=64, scale=0.1, dtype=gqa.BF16, kv_dtype=gqa.BF16, k_scale=None, v_scale=None,
                block_table=None, block_size=0, max_blocks=0, num_blocks=0, window=0, k_new=None,
                v_new=None, out=FAKE, workspace=None, workspace_bytes=0, num_splits=1)
    base.update(kw)
    for name, val in base.items():
        setattr(a, name, val)
    return a


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), Status.ERR_NULL),
    (dict(out=None), Status.ERR_NULL),
    (dict(seqlens=None), Status.ERR_NULL),
    (dict(k_new=FAKE), Status.ERR_NULL),                         # v_new missing
    (dict(kv_dtype=gqa.FP8_E4M3), Status.ERR_NULL),              # scales missing
    (dict(kv_dtype=gqa.FP8_E5M2), Status.ERR_NULL),              # scales missing
    (dict(kv_dtype=gqa.FP8_E5M2, k_scale=FAKE, v_scale=FAKE, T=17), Status.ERR_UNSUPPORTED),
    (dict(kv_dtype=4, k_scale=FAKE, v_scale=FAKE), Status.ERR_DTYPE),
    (dict(q=FAKE + 2), Status.ERR_ALIGN),
    (dict(k_new=FAKE + 8, v_new=FAKE), Status.ERR_ALIGN),
    (dict(T=0), Status.ERR_SHAPE),
    (dict(window=-1), Status.ERR_SHAPE),
    (dict(B=0), Status.ERR_SHAPE),
    (dict(Hq=524288, Hkv=524288), Status.ERR_SHAPE),                # 32 rows x 128 MiB > 2^31 - 1
    (dict(Hq=6, Hkv=4), Status.ERR_GROUP),
    (dict(d=32), Status.ERR_HEADDIM),
    (dict(dtype=gqa.F32), Status.ERR_DTYPE),
    (dict(kv_dtype=gqa.F32), Status.ERR_DTYPE),
    (dict(T=17, Hq=8, Hkv=2), Status.ERR_UNSUPPORTED),           # 17 tokens x group of 4 > 64 rows
    (dict(block_table=FAKE, block_size=8, max_blocks=8, num_blocks=8), Status.ERR_SHAPE),    # not a multiple of 16
    (dict(block_table=FAKE, block_size=24, max_blocks=3, num_blocks=8, Lmax=72), Status.ERR_SHAPE),
    (dict(block_table=FAKE, block_size=32, max_blocks=3, num_blocks=8), Status.ERR_SHAPE),  # Lmax != 96
    (dict(block_table=FAKE, block_size=32, max_blocks=2, num_blocks=0), Status.ERR_SHAPE),
    (dict(num_splits=65), Status.ERR_UNSUPPORTED),
    (dict(num_splits=2), Status.ERR_WORKSPACE),
    (dict(num_splits=2, workspace=FAKE, workspace_bytes=64), Status.ERR_WORKSPACE),
])
def test_decode_ex_validation(kw, expect):
    a = _ex_args(**kw)
    assert gqa.load().gqa_decode_ex(ctypes.byref(a), None) == expect


@pytest.mark.parametrize("B,T,Hq,Hkv,d,Lmax,ns", [(2, 2, 8, 2, 128, 64, 1), (2, 2, 8, 2, 128, 64, 2),
                                                  (3, 4, 32, 8, 64, 1000, 7), (1, 1, 4, 4, 128, 33, 33)])
def test_decode_ex_workspace_size(B, T, Hq, Hkv, d, Lmax, ns):
    a = _ex_args(B=B, T=T, Hq=Hq, Hkv=Hkv, d=d, Lmax=Lmax, num_splits=ns)
    got = ctypes.c_size_t(0)
    assert gqa.load().gqa_decode_ex_workspace_size(ctypes.byref(a), ctypes.byref(got)) == 0
    # pieces of ceil(Lmax / ns) keys rounded up to whole 32-key steps
    chunk = -(-Lmax // ns)
    chunk = -(-chunk // 32) * 32
    splits = -(-Lmax // chunk)
    want = 0 if splits == 1 else B * T * Hq * splits * (d + 2) * 4
    assert got.value == want


def test_decode_ex_struct_layout_matches_header(tmp_path):
    fields = [f[0] for f in DecodeExArgs._fields_]
    src = tmp_path / "layout.c"
    body = "".join('printf("%%s %%zu\\n", "%s", offsetof(gqa_decode_ex_args, %s));\n' % (f, f)
                   for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "gqa.h"\nint main(void){\n'
                   'printf("sizeof %zu\\n", sizeof(gqa_decode_ex_args));\n' + body + "return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                         check=True).stdout.splitlines())
    assert int(got["sizeof"]) == ctypes.sizeof(DecodeExArgs)
    for f in fields:
        assert int(got[f]) == getattr(DecodeExArgs, f).offset, f


@pytest.mark.parametrize("kw,expect", [
    (dict(window=-1), Status.ERR_SHAPE),
    (dict(window=16, causal=0), Status.ERR_UNSUPPORTED),
    (dict(q=None), Status.ERR_NULL),
    (dict(d=80), Status.ERR_HEADDIM),
    (dict(dt=gqa.F32), Status.ERR_DTYPE),
])
def test_prefill_ex_validation(kw, expect):
    a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, P=64, Hq=8, Hkv=2, d=128, causal=1, window=16,
             scale=0.1, dt=gqa.BF16, out=FAKE, stream=None)
    a.update(kw)
    st = gqa.load().gqa_prefill_ex(a["q"], a["k"], a["v"], a["B"], a["P"], a["Hq"], a["Hkv"],
                                   a["d"], a["causal"], a["window"], a["scale"], a["dt"], a["out"],
                                   a["stream"])
    assert st == expect


# --- binding: cache element codes (host logic, no device needed) ------------

def test_kv_code_mapping():
    import torch
    from gqa_kv_cache_amd._native import _kv_code
    u8 = torch.zeros(4, dtype=torch.uint8)
    assert _kv_code(u8, None) == gqa.FP8_E4M3
    assert _kv_code(u8, "e4m3") == gqa.FP8_E4M3
    assert _kv_code(u8, "e5m2") == gqa.FP8_E5M2
    assert _kv_code(u8.view(torch.float8_e5m2), None) == gqa.FP8_E5M2
    assert _kv_code(u8.view(torch.float8_e4m3fn), "e4m3") == gqa.FP8_E4M3
    assert _kv_code(torch.zeros(4, dtype=torch.bfloat16), None) == gqa.BF16
    with pytest.raises(TypeError):
        _kv_code(u8.view(torch.float8_e4m3fn), "e5m2")
    with pytest.raises(TypeError):
        _kv_code(torch.zeros(4, dtype=torch.bfloat16), "e4m3")
    with pytest.raises(ValueError):
        _kv_code(u8, "e3m4")
    with pytest.raises(TypeError):
        _kv_code(torch.zeros(4, dtype=torch.float16), None)
