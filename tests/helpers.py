"""Test-only helpers: widening stored inputs and comparing results."""
import numpy as np


def widen(a: np.ndarray) -> np.ndarray:
    """float32 values or uint16 bf16 bit patterns -> float64 (exact)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def to_lists(a: np.ndarray):
    return widen(a).tolist()


def bf16_tol_ok(got, ref, atol=2e-2, rtol=1e-2):
    """Elementwise |got - ref| <= atol + rtol * |ref| (bf16 inputs, fp32 accumulation)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    return bool(np.all(err <= atol + rtol * np.abs(ref))), float(err.max(initial=0.0))


def f32_tol_ok(got, ref, atol=1e-5):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return bool(np.all(err <= atol)), float(err.max(initial=0.0))
