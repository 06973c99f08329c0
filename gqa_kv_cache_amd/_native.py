"""ctypes binding of libgqa (the C ABI in include/gqa.h).

Argument marshalling only: shapes are read from the tensors, pointers and
the current HIP stream are passed through, and every step of the
computation runs in the library's HIP kernels.  PyTorch provides device
memory and streams.  There is no fallback: if the library is not built, or
a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import enum
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG, "libgqa.so")

F32, BF16 = 0, 1


class Status(enum.IntEnum):
    OK = 0
    ERR_NULL = 1
    ERR_SHAPE = 2
    ERR_GROUP = 3
    ERR_HEADDIM = 4
    ERR_DTYPE = 5
    ERR_ALIGN = 6
    ERR_WORKSPACE = 7
    ERR_UNSUPPORTED = 8
    ERR_HIP = 9


class GqaError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = Status(status) if status in Status._value2member_map_ else status
        msg = load().gqa_status_str(int(status)).decode()
        super().__init__((what + ": " if what else "") + msg)


_lib = None

EXPORTS = (
    "gqa_status_str", "gqa_decode", "gqa_decode_num_splits", "gqa_decode_workspace_size",
    "gqa_prefill", "gqa_kv_cache_elems", "gqa_decode_bytes", "gqa_decode_flops",
    "gqa_prefill_flops", "gqa_prefill_bytes",
)


def load():
    """Load libgqa.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY_PATH):
        raise RuntimeError("libgqa.so is not built (%s); build it with "
                           "`python -m gqa_kv_cache_amd.build`" % LIBRARY_PATH)
    lib = ctypes.CDLL(LIBRARY_PATH)
    vp, ci, cf, sz, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_uint64
    lib.gqa_status_str.argtypes = [ci]
    lib.gqa_status_str.restype = ctypes.c_char_p
    lib.gqa_decode.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp, vp, sz, ci, vp]
    lib.gqa_decode.restype = ci
    lib.gqa_decode_num_splits.argtypes = [ci, ci, ci, ci, ci, ci, ci, ctypes.POINTER(ci)]
    lib.gqa_decode_num_splits.restype = ci
    lib.gqa_decode_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci, ci, ctypes.POINTER(sz)]
    lib.gqa_decode_workspace_size.restype = ci
    lib.gqa_prefill.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, vp, vp]
    lib.gqa_prefill.restype = ci
    lib.gqa_kv_cache_elems.argtypes = [u64, u64, u64]
    lib.gqa_kv_cache_elems.restype = u64
    lib.gqa_decode_bytes.argtypes = [vp, ci, ci, ci, ci, ci]
    lib.gqa_decode_bytes.restype = u64
    lib.gqa_decode_flops.argtypes = [vp, ci, ci, ci]
    lib.gqa_decode_flops.restype = u64
    lib.gqa_prefill_flops.argtypes = [ci, ci, ci, ci, ci]
    lib.gqa_prefill_flops.restype = u64
    lib.gqa_prefill_bytes.argtypes = [ci, ci, ci, ci, ci, ci]
    lib.gqa_prefill_bytes.restype = u64
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().gqa_status_str(int(status)).decode()


def _check(st: int, what: str):
    if st != 0:
        raise GqaError(st, what)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("gqa: tensors must be float32 or bfloat16, got %s" % t.dtype)


def _require_cuda(name, t):
    if not t.is_cuda:
        raise ValueError("gqa: %s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("gqa: %s must be contiguous" % name)


def decode_num_splits(B, Hq, Hkv, d, Lmax, dtype_code, num_splits=0) -> int:
    out = ctypes.c_int(0)
    _check(load().gqa_decode_num_splits(B, Hq, Hkv, d, Lmax, dtype_code, num_splits,
                                        ctypes.byref(out)), "gqa_decode_num_splits")
    return out.value


def decode_workspace_size(B, Hq, Hkv, d, Lmax, dtype_code, num_splits=0) -> int:
    out = ctypes.c_size_t(0)
    _check(load().gqa_decode_workspace_size(B, Hq, Hkv, d, Lmax, dtype_code, num_splits,
                                            ctypes.byref(out)), "gqa_decode_workspace_size")
    return out.value


def decode(q, k_cache, v_cache, seqlens, scale=None, out=None, num_splits=0, workspace=None):
    """GQA decode step.  q [B,Hq,d]; k_cache, v_cache [B,Lmax,Hkv,d]; seqlens [B] int32.

    All tensors on one device; q, caches and out share one dtype (float32 or
    bfloat16).  Runs on the device's current stream; returns ``out``.
    """
    import torch
    lib = load()
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seqlens", seqlens)):
        _require_cuda(name, t)
    if seqlens.dtype != torch.int32:
        raise TypeError("gqa: seqlens must be int32")
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("gqa: expected q [B,Hq,d] and k_cache, v_cache [B,Lmax,Hkv,d]")
    B, Hq, d = q.shape
    Bk, Lmax, Hkv, dk = k_cache.shape
    if Bk != B or dk != d or tuple(seqlens.shape) != (B,):
        raise ValueError("gqa: inconsistent shapes")
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("gqa: q and the caches must share one dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require_cuda("out", out)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("gqa: out must match q in shape and dtype")
    with torch.cuda.device(q.device):
        need = decode_workspace_size(B, Hq, Hkv, d, Lmax, dt, num_splits)
        ws_ptr, ws_bytes = None, 0
        if need:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            _require_cuda("workspace", workspace)
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = lib.gqa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seqlens.data_ptr(),
                            B, Hq, Hkv, d, Lmax, float(scale), dt, out.data_ptr(), ws_ptr, ws_bytes,
                            int(num_splits), stream)
    _check(st, "gqa_decode")
    return out


def prefill(q, k, v, causal=True, scale=None, out=None):
    """GQA prefill.  q [B,P,Hq,d]; k, v [B,P,Hkv,d]; bfloat16.  Returns ``out``."""
    import torch
    lib = load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require_cuda(name, t)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("gqa: expected q [B,P,Hq,d] and k, v [B,P,Hkv,d]")
    B, P, Hq, d = q.shape
    Bk, Pk, Hkv, dk = k.shape
    if (Bk, Pk, dk) != (B, P, d):
        raise ValueError("gqa: inconsistent shapes")
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("gqa: q, k and v must share one dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require_cuda("out", out)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("gqa: out must match q in shape and dtype")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = lib.gqa_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, P, Hq, Hkv, d,
                             1 if causal else 0, float(scale), dt, out.data_ptr(), stream)
    _check(st, "gqa_prefill")
    return out


# --- counts --------------------------------------------------------------

def _host_i32(seqlens):
    arr = (ctypes.c_int32 * len(seqlens))(*[int(x) for x in seqlens])
    return arr


def kv_cache_elems(L, Hkv, d) -> int:
    return int(load().gqa_kv_cache_elems(int(L), int(Hkv), int(d)))


def decode_bytes(seqlens, Hq, Hkv, d, dtype_code) -> int:
    arr = _host_i32(seqlens)
    return int(load().gqa_decode_bytes(ctypes.addressof(arr), len(seqlens), Hq, Hkv, d, dtype_code))


def decode_flops(seqlens, Hq, d) -> int:
    arr = _host_i32(seqlens)
    return int(load().gqa_decode_flops(ctypes.addressof(arr), len(seqlens), Hq, d))


def prefill_flops(B, P, Hq, d, causal=True) -> int:
    return int(load().gqa_prefill_flops(B, P, Hq, d, 1 if causal else 0))


def prefill_bytes(B, P, Hq, Hkv, d, dtype_code) -> int:
    return int(load().gqa_prefill_bytes(B, P, Hq, Hkv, d, dtype_code))
