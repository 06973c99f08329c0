"""Test-only helpers moving seeded numpy inputs to the device and results back."""
import numpy as np
import torch

from tests.helpers import widen


def to_dev(a: np.ndarray, device="cuda"):
    """numpy float32 or uint16 (bf16 bits) -> device tensor (float32 / bfloat16)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def from_dev(t) -> np.ndarray:
    """device tensor -> float64 numpy (bf16 widened exactly)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return widen(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def bits(t) -> np.ndarray:
    """Raw bit patterns of a device tensor (for bitwise comparisons)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()
