"""Helpers shared by the GPU tests: host <-> device conversion and tolerance checks."""
from __future__ import annotations

import numpy as np
import torch

from synth import bf16_bits_to_f32


def to_dev(a: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    """numpy array (float32, or uint16 bf16 bit patterns) -> device tensor of that dtype."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a device tensor (uint16 for bf16, float32 otherwise)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def to_f64(t_or_a) -> np.ndarray:
    """Exact float64 value of a device tensor / host array (bf16 bit patterns widened)."""
    if isinstance(t_or_a, torch.Tensor):
        a = to_host_bits(t_or_a)
    else:
        a = t_or_a
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits); tiny floor near zero."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def attn_errors(got: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    """(max abs error, max abs error / max |ref|)."""
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    den = float(np.max(np.abs(ref))) if ref.size else 1.0
    return err, err / max(den, 1e-30)
