"""The entry point that allocates nothing: dion3_momentum_rowsel_noalloc keeps
the selection's partial sums in the library's fixed per-GPU scratch and must
give exactly what dion3_momentum_rowsel_ef gives with a caller's workspace
(M, indices, l1 keys and the selected sum of squares, bit for bit).  Two calls
in a row share the scratch, the second on a smaller input, so a stale partial
sum of the first call would show in the second.  Inputs too large for the
scratch are refused before anything is launched (CPU)."""

import ctypes

import numpy as np
import pytest
import torch

from muon_momentum_amd import synth

DEV = "cuda"


@pytest.fixture(scope="module")
def d():
    import muon_momentum_amd.dion3 as mod
    return mod


def _run(d, rows, cols, batch, k, step, noalloc, prev=None):
    M = synth.gradient(rows, cols, batch, dtype="bf16", device=DEV, group_seed=rows, step=step)
    G = synth.gradient(rows, cols, batch, dtype="bf16", device=DEV, group_seed=cols, step=step + 1)
    n, _, _ = d.dion3_canonical(d.make_group(M))
    idx = torch.full((batch, k), -1, dtype=torch.int32, device=DEV)
    keys = torch.empty(batch, n, dtype=torch.float64, device=DEV)
    sqn = torch.empty(batch, dtype=torch.float64, device=DEV)
    pk = prev.shape[1] if prev is not None else 0
    if noalloc:
        d.dion3_momentum_rowsel_noalloc(M, G, k, idx, keys, sqn, prev, pk, 0.95)
    else:
        d.dion3_momentum_rowsel_ef(M, G, k, idx, prev, pk, 0.95, keys, sqn)
    return M, idx, keys, sqn


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point(d):
    # first a large column-selected input (11008 x 4096: 11 row chunks of
    # partial sums), then a smaller row-selected one with a pending decay
    cases = [(11008, 4096, 6, 1024, None), (300, 1000, 2, 75, "prev")]
    for rows, cols, batch, k, prev in cases:
        pidx = None
        if prev:
            n = min(rows, cols)
            rng = np.random.default_rng(rows)
            pidx = torch.from_numpy(np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(batch)])
                                    .astype(np.int32)).to(DEV)
        want = _run(d, rows, cols, batch, k, 3, False, pidx)
        got = _run(d, rows, cols, batch, k, 3, True, pidx)
        torch.cuda.synchronize()
        for a, b in zip(want, got):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), (rows, cols)


def test_noalloc_refuses_inputs_beyond_the_scratch(d):
    """The partial sums of 40 column-selected 16384 x 8192 matrices need 80 MiB,
    more than the 64 MiB scratch: refused with DION3_ERR_TOO_LARGE before any
    launch (fake pointers are never touched)."""
    L = d.lib
    fake = ctypes.c_void_p(0x1000)
    big = d.Group(16384, 8192, 40, 16384 * 8192, d.BF16, -1)
    assert L.dion3_rowsel_workspace_bytes(ctypes.byref(big)) > (64 << 20)
    assert L.dion3_momentum_rowsel_noalloc(ctypes.byref(big), fake, fake, 16, fake, None, None, None, 0, 0.95,
                                           None) == -5
    assert b"fixed scratch" in L.dion3_status_string(-5)
    # invalid arguments are reported as such before the size check
    assert L.dion3_momentum_rowsel_noalloc(ctypes.byref(big), None, fake, 16, fake, None, None, None, 0, 0.95,
                                           None) == -1
