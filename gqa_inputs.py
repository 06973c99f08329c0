"""Seeded synthetic inputs for GQA decode and prefill.

This module serves both the GPU library's tests/benchmark and the CPU oracle.
It holds no attention arithmetic: only random draws, the rounding of those
draws to bf16, and the workload shapes.

Recipe (stable across runs, thread counts and machines):

* every tensor is drawn from numpy's PCG64 ``default_rng`` seeded with a list
  of integers ``[seed, tag]`` (q) or ``[seed, tag, b]`` (one stream per
  sequence b for K and V, and per sequence for prefill Q), with tags
  q=1, K=2, V=3; ragged lengths come from ``[seed, 0]``;
* values are ``standard_normal(dtype=float32)``, i.e. N(0, 1);
* bf16 tensors are the float32 draws rounded to nearest-even by integer bit
  arithmetic, stored as uint16 bit patterns;
* cache rows at or beyond ``seqlens[b]`` are never drawn: they hold NaN
  (``invalid="nan"``, parity runs, proving they are never read) or zero
  (``invalid="zero"``).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

TAG_LEN, TAG_Q, TAG_K, TAG_V = 0, 1, 2, 3
NAN_BF16 = np.uint16(0x7FC0)
NAN_F32_BITS = np.uint32(0x7FC00000)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs here are finite draws, so no NaN/Inf handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _draw(seed_words, shape, dtype: str) -> np.ndarray:
    rng = np.random.default_rng(list(seed_words))
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    raise ValueError(dtype)


def _storage(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def _fill_invalid(arr: np.ndarray, dtype: str, invalid: str) -> None:
    if invalid == "zero":
        arr[...] = 0
    elif invalid == "nan":
        if dtype == "f32":
            arr.view(np.uint32)[...] = NAN_F32_BITS
        else:
            arr[...] = NAN_BF16
    else:
        raise ValueError(invalid)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@dataclass
class DecodeCase:
    name: str
    q: np.ndarray          # [B, Hq, d]
    k: np.ndarray          # [B, Lmax, Hkv, d]
    v: np.ndarray          # [B, Lmax, Hkv, d]
    seqlens: np.ndarray    # [B] int32
    scale: float
    dtype: str             # "f32" or "bf16"
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, Hq, d = self.q.shape
        return dict(B=B, Hq=Hq, Hkv=self.k.shape[2], d=d, Lmax=self.k.shape[1])


@dataclass
class PrefillCase:
    name: str
    q: np.ndarray          # [B, P, Hq, d]
    k: np.ndarray          # [B, P, Hkv, d]
    v: np.ndarray          # [B, P, Hkv, d]
    causal: bool
    scale: float
    dtype: str
    meta: dict = field(default_factory=dict)


def decode_case(B, Hq, Hkv, d, Lmax, seqlens, dtype, q_seed, kv_seed, invalid="nan",
                scale=None, name="decode") -> DecodeCase:
    """q from [q_seed, 1]; K[b], V[b] rows < seqlens[b] from [kv_seed, 2|3, b]."""
    seqlens = np.asarray(seqlens, dtype=np.int32)
    assert seqlens.shape == (B,)
    st = _storage(dtype)
    q = _draw([q_seed, TAG_Q], (B, Hq, d), dtype)
    k = np.empty((B, Lmax, Hkv, d), st)
    v = np.empty((B, Lmax, Hkv, d), st)

    def one(b):
        n = int(seqlens[b])
        k[b, :n] = _draw([kv_seed, TAG_K, b], (n, Hkv, d), dtype)
        v[b, :n] = _draw([kv_seed, TAG_V, b], (n, Hkv, d), dtype)
        if n < Lmax:
            _fill_invalid(k[b, n:], dtype, invalid)
            _fill_invalid(v[b, n:], dtype, invalid)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(B)))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return DecodeCase(name, q, k, v, seqlens, float(scale), dtype,
                      dict(q_seed=q_seed, kv_seed=kv_seed, invalid=invalid))


def prefill_case(B, P, Hq, Hkv, d, dtype, seed, causal=True, scale=None,
                 name="prefill") -> PrefillCase:
    """Q[b], K[b], V[b] from [seed, 1|2|3, b]."""
    st = _storage(dtype)
    q = np.empty((B, P, Hq, d), st)
    k = np.empty((B, P, Hkv, d), st)
    v = np.empty((B, P, Hkv, d), st)

    def one(b):
        q[b] = _draw([seed, TAG_Q, b], (P, Hq, d), dtype)
        k[b] = _draw([seed, TAG_K, b], (P, Hkv, d), dtype)
        v[b] = _draw([seed, TAG_V, b], (P, Hkv, d), dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(B)))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return PrefillCase(name, q, k, v, bool(causal), float(scale), dtype, dict(seed=seed))


def prefill_growing_keys(B, P, Hq, Hkv, d, seed, profile, causal=True, name="prefill_growing") -> PrefillCase:
    """Prefill inputs whose key rows grow in magnitude along the prompt, so a
    row's largest score keeps rising and a lazily tracked softmax reference
    must move many times (the plain draws settle it on the first keys).

    profile: "linear" (key j scaled by 1 + 6 j / P), "exp" (by 2^(j / 96)), or
    "jump" (keys from P/2 on scaled by 64).  The scaled rows are rounded back
    to bf16; Q and V are the plain draws of prefill_case."""
    c = prefill_case(B, P, Hq, Hkv, d, "bf16", seed, causal=causal, name=name)
    j = np.arange(P, dtype=np.float64)
    if profile == "linear":
        f = 1.0 + 6.0 * j / P
    elif profile == "exp":
        f = np.exp2(j / 96.0)
    elif profile == "jump":
        f = np.where(j >= P // 2, 64.0, 1.0)
    else:
        raise ValueError(profile)
    k32 = (c.k.astype(np.uint32) << np.uint32(16)).view(np.float32)
    k32 = (k32 * f[None, :, None, None]).astype(np.float32)
    c.k[...] = bf16_bits_from_f32(k32)
    return c


# --------------------------------------------------------------------------
# The five workloads.
# --------------------------------------------------------------------------

def tiny_decode(hkv: int, invalid="nan") -> DecodeCase:
    """fp32, B=1, Hq=8, d=64, L=128; the same q for every hkv (2 = GQA, 8 = MHA, 1 = MQA)."""
    return decode_case(1, 8, hkv, 64, 128, [128], "f32", q_seed=1, kv_seed=10 + hkv,
                       invalid=invalid, name="tiny_fp32_B1_Hq8_Hkv%d_d64_L128" % hkv)


def decode_70b(invalid="zero") -> DecodeCase:
    """70B-class layer decode: bf16, B=32, Hq=64, Hkv=8, d=128, every sequence at L=4096."""
    return decode_case(32, 64, 8, 128, 4096, [4096] * 32, "bf16", q_seed=2, kv_seed=2,
                       invalid=invalid, name="decode_bf16_B32_Hq64_Hkv8_d128_L4096")


SWEEP_HKV = (64, 16, 8, 4, 1)


def sweep_decode(hkv: int, invalid="zero") -> DecodeCase:
    """Head-sharing sweep: bf16, B=16, Hq=64, d=128, L=2048; one q for every hkv."""
    return decode_case(16, 64, hkv, 128, 2048, [2048] * 16, "bf16", q_seed=3, kv_seed=30 + hkv,
                       invalid=invalid, name="sweep_bf16_B16_Hq64_Hkv%d_d128_L2048" % hkv)


def ragged_seqlens(B=64, Lmax=32768, seed=4) -> np.ndarray:
    rng = np.random.default_rng([seed, TAG_LEN])
    return rng.integers(1, Lmax + 1, B).astype(np.int32)


def ragged_decode(invalid="nan") -> DecodeCase:
    """Ragged batch: bf16, B=64, Hq=32, Hkv=8, d=128, Lmax=32768, seqlens ~ U[1, 32768]."""
    sl = ragged_seqlens()
    return decode_case(64, 32, 8, 128, 32768, sl, "bf16", q_seed=4, kv_seed=4, invalid=invalid,
                       name="ragged_bf16_B64_Hq32_Hkv8_d128_Lmax32768")


def prefill_causal() -> PrefillCase:
    """Causal prefill: bf16, B=2, P=4096, Hq=32, Hkv=8, d=128."""
    return prefill_case(2, 4096, 32, 8, 128, "bf16", seed=5, causal=True,
                        name="prefill_bf16_B2_P4096_Hq32_Hkv8_d128_causal")


# --------------------------------------------------------------------------
# Extended decode inputs (several new tokens, appended rows, FP8 rows, paged
# pools, windows).  Draws only; the layouts are the ones the extended decode
# call takes.
# --------------------------------------------------------------------------

TAG_KNEW, TAG_VNEW, TAG_SCALE, TAG_PERM = 4, 5, 6, 7
NAN_E4M3 = np.uint8(0x7F)
NAN_E5M2 = np.uint8(0x7F)      # S.11111.11: a NaN in E5M2 as well


def _draw_e4m3(seed_words, shape) -> np.ndarray:
    """Random OCP E4M3 codes: random sign and mantissa, exponent field drawn
    from 3..10 (magnitudes 2^-4 .. 15), so no NaN and no subnormal patterns."""
    rng = np.random.default_rng(list(seed_words))
    sign = rng.integers(0, 2, shape, dtype=np.uint8) << np.uint8(7)
    expo = rng.integers(3, 11, shape, dtype=np.uint8) << np.uint8(3)
    mant = rng.integers(0, 8, shape, dtype=np.uint8)
    return (sign | expo | mant).astype(np.uint8)


def _draw_e5m2(seed_words, shape) -> np.ndarray:
    """Random OCP E5M2 codes: random sign and mantissa, exponent field drawn
    from 11..18 (magnitudes 2^-4 .. 14), so no infinity, NaN or subnormal."""
    rng = np.random.default_rng(list(seed_words))
    sign = rng.integers(0, 2, shape, dtype=np.uint8) << np.uint8(7)
    expo = rng.integers(11, 19, shape, dtype=np.uint8) << np.uint8(2)
    mant = rng.integers(0, 4, shape, dtype=np.uint8)
    return (sign | expo | mant).astype(np.uint8)


FP8_KINDS = {"fp8": "e4m3", "e5m2": "e5m2"}   # case kind -> FP8 format of its byte rows


@dataclass
class DecodeExCase:
    name: str
    q: np.ndarray            # [B, T, Hq, d]
    k: np.ndarray            # cache after the append: [B, Lmax, Hkv, d] or pool [nb, bs, Hkv, d]
    v: np.ndarray
    k_pre: np.ndarray        # same cache before the append: rows of the new tokens hold NaN
    v_pre: np.ndarray
    k_new: np.ndarray        # [B, T, Hkv, d], the rows the append stores
    v_new: np.ndarray
    seqlens: np.ndarray      # [B] int32, counts the T new tokens
    scale: float
    dtype: str               # q/out dtype: "f32" or "bf16"
    kv: str                  # "same" (q's dtype), "fp8" (E4M3 bytes) or "e5m2" (E5M2 bytes)
    k_scale: np.ndarray = None   # [Hkv] float32 (FP8 kinds only)
    v_scale: np.ndarray = None
    block_table: np.ndarray = None   # [B, max_blocks] int32 (paged only)
    block_size: int = 0
    window: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def T(self):
        return self.q.shape[1]

    @property
    def kv_format(self):
        """FP8 format of the byte rows ("e4m3" / "e5m2"), None for q's dtype."""
        return FP8_KINDS.get(self.kv)


def decode_ex_case(B, T, Hq, Hkv, d, Lmax, seqlens, dtype, seed, kv="same", paged=False,
                   block_size=64, window=0, invalid="nan", scale=None,
                   name="decode_ex") -> DecodeExCase:
    """q from [seed, 1]; cached rows of sequence b from [seed, 2|3, b]; the T
    new rows from [seed, 4|5]; FP8 per-head scales from [seed, 6]; the block
    permutation of a paged pool from [seed, 7].  kv: "same", "fp8" (E4M3
    bytes) or "e5m2" (E5M2 bytes)."""
    seqlens = np.asarray(seqlens, dtype=np.int32)
    assert seqlens.shape == (B,) and int(seqlens.min()) >= T and int(seqlens.max()) <= Lmax
    assert kv in ("same", "fp8", "e5m2")
    fp8 = kv != "same"
    st = np.uint8 if fp8 else _storage(dtype)

    def rows(words, shape):
        if kv == "e5m2":
            return _draw_e5m2(words, shape)
        return _draw_e4m3(words, shape) if fp8 else _draw(words, shape, dtype)

    def poison(a):
        if fp8:
            a[...] = (NAN_E5M2 if kv == "e5m2" else NAN_E4M3) if invalid == "nan" else 0
        else:
            _fill_invalid(a, dtype, invalid)

    q = _draw([seed, TAG_Q], (B, T, Hq, d), dtype)
    kc = np.empty((B, Lmax, Hkv, d), st)
    vc = np.empty((B, Lmax, Hkv, d), st)
    k_new = rows([seed, TAG_KNEW], (B, T, Hkv, d))
    v_new = rows([seed, TAG_VNEW], (B, T, Hkv, d))
    for b in range(B):
        n = int(seqlens[b])
        kc[b, :n - T] = rows([seed, TAG_K, b], (n - T, Hkv, d))
        vc[b, :n - T] = rows([seed, TAG_V, b], (n - T, Hkv, d))
        poison(kc[b, n - T:])
        poison(vc[b, n - T:])
    k_pre, v_pre = kc.copy(), vc.copy()
    for b in range(B):
        n = int(seqlens[b])
        kc[b, n - T:n] = k_new[b]
        vc[b, n - T:n] = v_new[b]

    k_scale = v_scale = None
    if fp8:
        rng = np.random.default_rng([seed, TAG_SCALE])
        k_scale = rng.uniform(0.05, 0.4, Hkv).astype(np.float32)
        v_scale = rng.uniform(0.05, 0.4, Hkv).astype(np.float32)

    block_table = None
    if paged:
        assert Lmax % block_size == 0
        maxb = Lmax // block_size
        nblocks = B * maxb + 3           # a few pool blocks no sequence uses
        perm = np.random.default_rng([seed, TAG_PERM]).permutation(nblocks)[: B * maxb]
        block_table = perm.reshape(B, maxb).astype(np.int32)

        def to_pool(c):
            pool = np.empty((nblocks, block_size, Hkv, d), st)
            poison(pool)
            for b in range(B):
                for i in range(maxb):
                    pool[block_table[b, i]] = c[b, i * block_size:(i + 1) * block_size]
            return pool

        kc, vc, k_pre, v_pre = to_pool(kc), to_pool(vc), to_pool(k_pre), to_pool(v_pre)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return DecodeExCase(name, q, kc, vc, k_pre, v_pre, k_new, v_new, seqlens, float(scale), dtype,
                        kv, k_scale, v_scale, block_table, block_size if paged else 0, int(window),
                        dict(seed=seed, paged=paged, invalid=invalid))
