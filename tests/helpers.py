"""Shared helpers for the GPU parity tests (no method arithmetic here: the
step helper only calls the library's entry points)."""

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


def manual_step(d, groups, ks, params, eta, wd, mu, keep=None):
    """The step through the individual entry points, batched like dion3_step
    (groups of equal canonical (k, m) share one Newton-Schulz call; a square
    class uses standard Newton-Schulz).  Returns
    per-group idx and the Newton-Schulz output O (canonical orientation) of
    every matrix, or, with keep = {group: [matrix, ...]}, of those only."""
    ns_t = d.torch_dtype(params.ns_dtype)
    classes = {}
    for gi, (W, M, G) in enumerate(groups):
        n, m, ax = d.dion3_canonical(d.make_group(M))
        classes.setdefault((ks[gi], m), []).append(gi)
    idxs, Os = [None] * len(groups), [None] * len(groups)
    for (k, m), members in classes.items():
        nb = sum(groups[g][0].shape[0] for g in members)
        X = torch.empty(nb, k, m, dtype=ns_t, device="cuda")
        Ob = torch.empty_like(X)
        off = 0
        for g in members:
            W, M, G = groups[g]
            b = M.shape[0]
            idx = torch.empty(b, k, dtype=torch.int32, device="cuda")
            sqn = torch.empty(b, dtype=torch.float64, device="cuda")
            d.dion3_momentum_rowsel(M, G, k, idx, None, sqn)
            d.dion3_gather_rows(M, idx, k, sqn, X[off:off + b], eps=params.eps)
            idxs[g] = idx
            off += b
        # like the whole step: standard Newton-Schulz when the class is square
        if k == m:
            d.dion3_standard_ns(X, Ob, params)
        else:
            d.dion3_gram_ns_gathered(X, Ob, params)
        off = 0
        for g in members:
            W, M, G = groups[g]
            b = M.shape[0]
            d.dion3_apply_rows(W, M, idxs[g], k, Ob[off:off + b], eta, wd, mu)
            if keep is None:
                Os[g] = Ob[off:off + b].clone()
            else:
                Os[g] = {j: Ob[off + j].clone() for j in keep.get(g, [])}
            off += b
    torch.cuda.synchronize()
    return idxs, Os
