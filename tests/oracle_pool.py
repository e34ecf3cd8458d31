"""Oracle checks of whole matrices in worker processes (CPU only).

The workers are started with the "spawn" method and import only NumPy and the
oracle, so they never touch the GPU; the parent hands them host copies of the
GPU's inputs and results as raw bit patterns.  Used by the full-size parity
tests, where the oracle's exact rounding of every element of a 7B-shaped set
takes minutes of CPU time on one core.
"""

from __future__ import annotations

import math
import multiprocessing as mp
import os

import numpy as np

import oracle as O

# 2^30: a row of at most 2^22 bf16 values whose nonzero magnitudes span less
# than this ratio has an exact fp64 sum (every value is a multiple of the
# smallest value's unit in the last place, and the total stays below 2^53 of
# those units), so np.sum gives the correctly rounded l1 norm
_EXACT_SPAN = 2.0 ** 30


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (int16 / uint16) to their exact fp64 values."""
    u = bits.astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns of fp64 values that are exact bf16 values."""
    f = x.astype(np.float32)                       # exact for bf16 values
    return (f.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)


def exact_l1(M: np.ndarray) -> np.ndarray:
    """Correctly rounded l1 norm of every row: np.sum where the row's dynamic
    range makes the fp64 sum exact, the oracle's math.fsum otherwise."""
    A = np.abs(M)
    keys = A.sum(axis=1)
    mx = A.max(axis=1)
    nz = np.where(A > 0, A, np.inf).min(axis=1)
    slow = (mx > 0) & ((mx / nz >= _EXACT_SPAN) | (M.shape[1] > (1 << 22)))
    for i in np.nonzero(slow)[0]:
        keys[i] = O.l1_row_norms(M[i][None])[0]
    return keys


def check_two_steps(task):
    """Two steps of the Dion3 momentum and selection from M0 = 0, on one matrix
    in canonical orientation, against the GPU's selections and final momentum.

    task = (key, G1 bits, G2 bits, GPU M after the second step's decay bits,
    GPU idx of step 1, GPU idx of step 2, k, mu).  Returns (key, None) or
    (key, what differs)."""
    key, g1, g2, m2, idx1, idx2, k, mu = task
    mu32 = O.f32(mu)
    G1 = bf16_bits_to_f64(g1)
    # step 1 from M0 = 0: the oracle's momentum is round(0 + g) = g exactly
    M1 = G1
    s1 = O.select_rows(exact_l1(M1), k)
    if not np.array_equal(s1, idx1):
        return key, "idx step 1"
    M1 = M1.copy()
    M1[s1] = O.round_to(mu32 * M1[s1], "bf16")        # error feedback of step 1
    M2 = O.momentum_accumulate(M1, bf16_bits_to_f64(g2), "bf16")
    s2 = O.select_rows(exact_l1(M2), k)
    if not np.array_equal(s2, idx2):
        return key, "idx step 2"
    M2[s2] = O.round_to(mu32 * M2[s2], "bf16")        # error feedback of step 2
    if not np.array_equal(f64_to_bf16_bits(M2), m2):
        return key, "M after step 2"
    return key, None


def pool(workers: int | None = None):
    """A spawn-context process pool sized to the machine's CPU share (at most
    15 workers)."""
    n = workers or max(1, min(15, (os.cpu_count() or 2) - 1))
    return mp.get_context("spawn").Pool(n)
