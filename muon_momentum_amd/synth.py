"""Seeded synthetic inputs with the shapes of transformer weight sets.

This module only draws random numbers; it holds none of the optimizer's
arithmetic.  Tests and the benchmark use it to build the same inputs for the
HIP library and for the CPU oracle (the oracle reads host copies of the same
bits, so no generator has to be reproduced on the other side).

Recipe (stands in for gradients of dense transformers trained on synthetic
data):
  * gradient G = z * s, z ~ N(0, 1) drawn fresh each step, s ~ LogNormal(0, 1)
    one scale per line of the selection axis (rows when rows <= cols, columns
    otherwise), fixed per matrix; computed in fp32, rounded once to storage.
  * weights W0 ~ N(0, 0.02^2) rounded to storage; momentum M0 = 0.
  * same-shape matrices are packed into one [batch, rows, cols] tensor.
"""

from __future__ import annotations

import torch

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

# Shape sets: per layer, (rows, cols, count).  Up/gate are hidden x ffn,
# down is ffn x hidden (the stored orientation decides the selection axis).
SHAPE_SETS = {
    "1b": {"layers": 16, "shapes": [(2048, 2048, 4), (2048, 8192, 2), (8192, 2048, 1)]},
    "7b": {"layers": 32, "shapes": [(4096, 4096, 4), (4096, 11008, 2), (11008, 4096, 1)]},
    "14b": {"layers": 40, "shapes": [(5120, 5120, 4), (5120, 13824, 2), (13824, 5120, 1)]},
}


def shape_groups(name: str):
    """[(rows, cols, batch)] for a shape set: every same-shape matrix in one group."""
    s = SHAPE_SETS[name]
    return [(r, c, s["layers"] * cnt) for r, c, cnt in s["shapes"]]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed & 0x7FFFFFFFFFFFFFFF)
    return g


def _scale_axis(rows: int, cols: int, sel_axis: int) -> int:
    if sel_axis in (0, 1):
        return sel_axis
    return 0 if rows <= cols else 1


def gradient(rows: int, cols: int, batch: int, *, dtype: str = "bf16", device="cpu",
             group_seed: int = 0, step: int = 0, sel_axis: int = -1,
             scale_axis: int | None = None) -> torch.Tensor:
    """G[b] = z * s for b in range(batch): fresh z per step, fixed s per matrix.

    `scale_axis` (default: the selection axis) says which lines carry the
    log-normal scales; scale_axis=0 on a column-selected matrix gives the
    near-tie stress case (all column norms close)."""
    ax = _scale_axis(rows, cols, sel_axis) if scale_axis is None else scale_axis
    out = torch.empty(batch, rows, cols, dtype=TORCH_DTYPES[dtype], device=device)
    for b in range(batch):
        mat_id = group_seed * 100003 + b
        gs = _gen(0x5CA1E000 + mat_id, device)
        nlines = rows if ax == 0 else cols
        s = torch.exp(torch.randn(nlines, generator=gs, device=device, dtype=torch.float32))
        gz = _gen(0x6A7D0000 + 1000 * step + mat_id * 7919, device)
        z = torch.randn(rows, cols, generator=gz, device=device, dtype=torch.float32)
        z *= s[:, None] if ax == 0 else s[None, :]
        out[b].copy_(z)
    return out


def weights(rows: int, cols: int, batch: int, *, dtype: str = "bf16", device="cpu",
            group_seed: int = 0, std: float = 0.02) -> torch.Tensor:
    out = torch.empty(batch, rows, cols, dtype=TORCH_DTYPES[dtype], device=device)
    for b in range(batch):
        g = _gen(0x3E1670 + group_seed * 100003 + b, device)
        out[b].copy_(torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32) * std)
    return out


def symmetric(n: int, batch: int, *, dtype: str = "f16", device="cpu", seed: int = 1) -> torch.Tensor:
    """(A + A^T)/sqrt(2) with A entries N(0, 1/n): a symmetric test operand."""
    g = _gen(0x5E3 + seed, device)
    a = torch.randn(batch, n, n, generator=g, device=device, dtype=torch.float32) / (n ** 0.5)
    return ((a + a.transpose(1, 2)) * (0.5 ** 0.5)).to(TORCH_DTYPES[dtype])


def dense(rows: int, cols: int, batch: int, *, dtype: str = "f16", device="cpu",
          seed: int = 1, std: float | None = None) -> torch.Tensor:
    """Entries N(0, std^2), std defaulting to 1/sqrt(cols)."""
    g = _gen(0xDE45E + seed, device)
    sd = (1.0 / cols ** 0.5) if std is None else std
    a = torch.randn(batch, rows, cols, generator=g, device=device, dtype=torch.float32) * sd
    return a.to(TORCH_DTYPES[dtype])
