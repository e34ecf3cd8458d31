"""Shared helpers for the GPU parity tests (no method arithmetic here)."""

import numpy as np
import torch


def to64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a float tensor (bf16/f16/f32 all embed exactly)."""
    return t.detach().to("cpu").to(torch.float32 if t.dtype != torch.float64 else torch.float64).numpy().astype(np.float64)


def rel_fro(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a tensor, for bit-exact comparisons."""
    t = t.detach().to("cpu").contiguous()
    view = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.float16: torch.int16,
            torch.float64: torch.int64}[t.dtype]
    return t.view(view).numpy()


def np_bits(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Bit patterns of fp64 values that are exactly representable in dtype."""
    return bits(torch.from_numpy(np.asarray(x, dtype=np.float64)).to(dtype))
