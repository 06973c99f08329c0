"""ctypes front end of the fp64 C oracle (``gqa_oracle.c``).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU
baseline use this module.  The product library never imports it.

Inputs are numpy arrays exactly as the GPU receives them: float32 values, or
bf16 bit patterns stored as uint16.  The C code widens every element exactly
to double and returns double results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

_lib = None


def build(force: bool = False) -> str:
    """Compile gqa_oracle.c into liboracle.so with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    i64, vp, dbl, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
    lib.oracle_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, dbl, ci, vp, i64, vp]
    lib.oracle_decode.restype = ci
    lib.oracle_decode_weights.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, dbl, ci,
                                          i64, i64, vp, vp]
    lib.oracle_decode_weights.restype = ci
    lib.oracle_prefill.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ci, dbl, ci, vp, i64, vp]
    lib.oracle_prefill.restype = ci
    lib.oracle_mha_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, dbl, ci, vp]
    lib.oracle_mha_decode.restype = ci
    lib.oracle_mqa_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, dbl, ci, vp]
    lib.oracle_mqa_decode.restype = ci
    lib.oracle_decode_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, dbl, ci, ci,
                                     vp, vp, vp, i64, i64, i64, vp, i64, vp, vp]
    lib.oracle_decode_ex.restype = ci
    lib.oracle_append.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, i64, i64]
    lib.oracle_append.restype = ci
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint]
    lib.oracle_e4m3_value.restype = dbl
    lib.oracle_e5m2_value.argtypes = [ctypes.c_uint]
    lib.oracle_e5m2_value.restype = dbl
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ci
    lib.oracle_set_threads.argtypes = [ci]
    lib.oracle_set_threads.restype = ci
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def swap_library(path):
    """Point this module at another build of the oracle (used by the mutation
    tests, which compile deliberately broken copies); returns the previous
    handle, or None.  Pass None to restore the default on next use."""
    global _lib
    prev = _lib
    _lib = None if path is None else _bind(ctypes.CDLL(path))
    return prev


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 values or uint16 bf16 bit patterns, got %s" % a.dtype)


def _c(a: np.ndarray) -> np.ndarray:
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("oracle inputs must be C-contiguous")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


class OracleError(RuntimeError):
    pass


def num_threads() -> int:
    """OpenMP threads the oracle runs on (OMP_NUM_THREADS or all cores)."""
    return _load().oracle_num_threads()


def set_threads(n: int) -> int:
    """Run later oracle calls on n OpenMP threads; returns the previous count."""
    return _load().oracle_set_threads(int(n))


def decode(q, k, v, seqlens, scale, rows=None) -> np.ndarray:
    """GQA decode.  q [B,Hq,d]; k, v [B,Lmax,Hkv,d]; seqlens [B] int.

    Returns [B,Hq,d] float64, or [len(rows),d] when ``rows`` (flat b*Hq+h
    indices) is given.
    """
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dtype_code(q)
    assert _dtype_code(k) == dt and _dtype_code(v) == dt
    B, Hq, d = q.shape
    Bk, Lmax, Hkv, dk = k.shape
    assert Bk == B and dk == d and v.shape == k.shape
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    assert sl.shape == (B,)
    if rows is None:
        out = np.empty((B, Hq, d), np.float64)
        r, nrows = None, B * Hq
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((r.size, d), np.float64)
        nrows = r.size
    rc = _load().oracle_decode(q.ctypes.data, k.ctypes.data, v.ctypes.data, sl.ctypes.data,
                               B, Hq, Hkv, d, Lmax, float(scale), dt, _ptr(r), nrows,
                               out.ctypes.data)
    if rc:
        raise OracleError("oracle_decode returned %d" % rc)
    return out


def decode_weights(q, k, v, seqlens, scale, b, h):
    """(weights[seqlens[b]], out[d]) of decode row (b, h); weights are normalised."""
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dtype_code(q)
    B, Hq, d = q.shape
    _, Lmax, Hkv, _ = k.shape
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    w = np.empty(max(int(sl[b]), 1), np.float64)
    out = np.empty(d, np.float64)
    rc = _load().oracle_decode_weights(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                       sl.ctypes.data, B, Hq, Hkv, d, Lmax, float(scale), dt,
                                       int(b), int(h), w.ctypes.data, out.ctypes.data)
    if rc:
        raise OracleError("oracle_decode_weights returned %d" % rc)
    return w[: int(sl[b])], out


def prefill(q, k, v, causal, scale, rows=None) -> np.ndarray:
    """GQA prefill.  q [B,P,Hq,d]; k, v [B,P,Hkv,d].

    Returns [B,P,Hq,d] float64, or [len(rows),d] for flat (b*P+i)*Hq+h rows.
    """
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dtype_code(q)
    assert _dtype_code(k) == dt and _dtype_code(v) == dt
    B, P, Hq, d = q.shape
    Bk, Pk, Hkv, dk = k.shape
    assert (Bk, Pk, dk) == (B, P, d) and v.shape == k.shape
    if rows is None:
        out = np.empty((B, P, Hq, d), np.float64)
        r, nrows = None, B * P * Hq
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((r.size, d), np.float64)
        nrows = r.size
    rc = _load().oracle_prefill(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, P, Hq, Hkv, d,
                                1 if causal else 0, float(scale), dt, _ptr(r), nrows,
                                out.ctypes.data)
    if rc:
        raise OracleError("oracle_prefill returned %d" % rc)
    return out


def mha_decode(q, k, v, seqlens, scale) -> np.ndarray:
    """Multi-head attention decode (k, v have exactly Hq heads)."""
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dtype_code(q)
    B, H, d = q.shape
    assert k.shape[2] == H and k.shape[3] == d
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    out = np.empty((B, H, d), np.float64)
    rc = _load().oracle_mha_decode(q.ctypes.data, k.ctypes.data, v.ctypes.data, sl.ctypes.data,
                                   B, H, d, k.shape[1], float(scale), dt, out.ctypes.data)
    if rc:
        raise OracleError("oracle_mha_decode returned %d" % rc)
    return out


def mqa_decode(q, k, v, seqlens, scale) -> np.ndarray:
    """Multi-query attention decode (k, v have exactly one head)."""
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dtype_code(q)
    B, H, d = q.shape
    assert k.shape[2] == 1 and k.shape[3] == d
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    out = np.empty((B, H, d), np.float64)
    rc = _load().oracle_mqa_decode(q.ctypes.data, k.ctypes.data, v.ctypes.data, sl.ctypes.data,
                                   B, H, d, k.shape[1], float(scale), dt, out.ctypes.data)
    if rc:
        raise OracleError("oracle_mqa_decode returned %d" % rc)
    return out


def e4m3_value(byte: int) -> float:
    """Value of one OCP FP8 E4M3 byte (NaN for the S.1111.111 patterns)."""
    return _load().oracle_e4m3_value(int(byte) & 0xFF)


def e5m2_value(byte: int) -> float:
    """Value of one OCP FP8 E5M2 byte (+-inf for S.11111.00, NaN for S.11111.mm, mm != 0)."""
    return _load().oracle_e5m2_value(int(byte) & 0xFF)


_KV_FORMATS = {"e4m3": 1, "e5m2": 2}


def decode_ex(q, k, v, seqlens, scale, *, k_scale=None, v_scale=None, block_table=None,
              block_size=0, window=0, rows=None, kv_format="e4m3", terms=False):
    """Extended GQA decode.  q [B,T,Hq,d] (fp32 or bf16 bits).

    k, v: contiguous [B,Lmax,Hkv,d] or, with ``block_table`` [B,max_blocks],
    a paged pool [nblocks,block_size,Hkv,d]; stored in q's dtype, or as FP8
    bytes (uint8) in ``kv_format`` ("e4m3" or "e5m2") scaled per KV head by
    ``k_scale``/``v_scale`` [Hkv].
    seqlens [B] counts the T new tokens; token t sits at seqlens[b]-T+t.
    window > 0 keeps the last ``window`` keys of every token.  Returns
    [B,T,Hq,d] float64, or [len(rows),d] for flat ((b*T+t)*Hq+h) rows.

    terms=True also returns the error-model terms of every output row, for
    the tests' derived tolerances: (out, sigma, mu, kappa) with sigma, mu
    shaped like out and kappa one value per row (out's shape without d):
    sigma_c = sum_j w_j |v_jc - out_c|, mu_c = sum_j w_j |v_jc| (w the
    normalised softmax weights of the row's visible keys), kappa =
    |scale| * max_j sum_c |q_c| |k_jc|.  ``out`` is the same either way.
    """
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dtype_code(q)
    B, T, Hq, d = q.shape
    fmt = _KV_FORMATS[kv_format] if k.dtype == np.uint8 else 0
    if fmt:
        assert v.dtype == np.uint8 and k_scale is not None and v_scale is not None
    else:
        assert _dtype_code(k) == dt and _dtype_code(v) == dt
    assert v.shape == k.shape and k.shape[3] == d
    Hkv = k.shape[2]
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    assert sl.shape == (B,)
    if block_table is None:
        assert k.shape[0] == B
        Lmax, bt, maxb, bs = k.shape[1], None, 0, 0
    else:
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        assert bt.shape[0] == B and k.shape[1] == block_size
        maxb, bs = bt.shape[1], int(block_size)
        Lmax = maxb * bs
        assert bt.min() >= 0 and bt.max() < k.shape[0]
    ks = None if k_scale is None else np.ascontiguousarray(k_scale, dtype=np.float32)
    vs = None if v_scale is None else np.ascontiguousarray(v_scale, dtype=np.float32)
    if rows is None:
        out = np.empty((B, T, Hq, d), np.float64)
        r, nrows = None, B * T * Hq
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((r.size, d), np.float64)
        nrows = r.size
    tm = np.empty((nrows, 2 * d + 1), np.float64) if terms else None
    rc = _load().oracle_decode_ex(q.ctypes.data, k.ctypes.data, v.ctypes.data, sl.ctypes.data,
                                  B, T, Hq, Hkv, d, Lmax, float(scale), dt, fmt,
                                  _ptr(ks), _ptr(vs), _ptr(bt), maxb, bs, int(window), _ptr(r),
                                  nrows, out.ctypes.data, _ptr(tm))
    if rc:
        raise OracleError("oracle_decode_ex returned %d" % rc)
    if not terms:
        return out
    shape = out.shape
    return (out, tm[:, :d].reshape(shape), tm[:, d:2 * d].reshape(shape),
            tm[:, 2 * d].reshape(shape[:-1]))


def append(k_cache, v_cache, k_new, v_new, seqlens, *, block_table=None, block_size=0):
    """Store k_new/v_new [B,T,Hkv,d] at rows seqlens[b]-T+t of the caches, in place.

    The caches are contiguous [B,Lmax,Hkv,d] or paged pools as in decode_ex;
    rows are copied byte for byte (same element type as the cache).
    """
    k_cache, v_cache, k_new, v_new = _c(k_cache), _c(v_cache), _c(k_new), _c(v_new)
    assert k_cache.dtype == k_new.dtype == v_cache.dtype == v_new.dtype
    B, T, Hkv, d = k_new.shape
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    if block_table is None:
        Lmax, bt, maxb, bs = k_cache.shape[1], None, 0, 0
    else:
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        maxb, bs = bt.shape[1], int(block_size)
        Lmax = maxb * bs
    rc = _load().oracle_append(k_cache.ctypes.data, v_cache.ctypes.data, k_new.ctypes.data,
                               v_new.ctypes.data, sl.ctypes.data, B, T, Hkv, d, Lmax,
                               k_cache.itemsize, _ptr(bt), maxb, bs)
    if rc:
        raise OracleError("oracle_append returned %d" % rc)
