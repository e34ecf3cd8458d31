"""Parity of the benchmarked call at the full size of the 7B shape set.

The benchmark times StepPlan.step_deferred: dion3_step_deferred on three
streams (the Newton-Schulz products on one, the overlapped memory passes on a
compute-unit-limited one, the caller's stream), with the error-feedback decay
of each step's selection applied by the next step's momentum pass.  Here that
exact call runs two steps of the 7B set at f = 1/4 and is compared

  * with the same two steps through the single-stream entry points
    (helpers.manual_step, decay applied right after each update): selected
    indices and W after each step, and M once the pending decay is completed,
    bit for bit on every matrix of every group;
  * with the oracle on every matrix: selected indices of both steps and the
    final momentum, bit for bit ("Dion3: Full-Stack Orthogonal Updates",
    Section 6: top-k l1 selection; error feedback M <- mu M_hat + (M - M_hat)
    is exact, so indices and momentum never depend on the fp16 iteration).

The oracle's exact rounding of the 6.5 G momentum entries runs in a pool of
CPU worker processes (tests/oracle_pool.py)."""

import math
import sys

import numpy as np
import pytest
import torch

from helpers import manual_step
from muon_momentum_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def d():
    import muon_momentum_amd.dion3 as mod
    return mod


def _bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy()


@pytest.mark.timeout(900)
def test_7b_benchmarked_call_every_matrix(d):
    import oracle_pool as P

    groups = synth.shape_groups("7b")
    f, mu = 0.25, 0.95
    eta = 0.02 / math.sqrt(f)
    ks = [d.dion3_k_from_fraction(min(r, c), f) for r, c, _ in groups]
    params = d.make_ns_params(ns_dtype=d.F16)
    A, B, G1 = [], [], []
    for gi, (r, c, b) in enumerate(groups):
        W = synth.weights(r, c, b, dtype="bf16", device=DEV, group_seed=gi)
        G = synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=gi, step=0)
        A.append([W, torch.zeros_like(W), G.clone()])
        B.append([W.clone(), torch.zeros_like(W), G.clone()])
        G1.append(G)
    idx_a = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(groups, ks)]
    plan = d.StepPlan([g[0] for g in A], [g[1] for g in A], [g[2] for g in A], ks, idx_a, params)
    idx1 = []
    for step in range(2):
        if step:
            for gi, (r, c, b) in enumerate(groups):
                Gn = synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=gi, step=1)
                A[gi][2].copy_(Gn)
                B[gi][2].copy_(Gn)
                del Gn
        plan.step_deferred(eta, 0.0, mu, has_prev=step > 0)          # the benchmarked call
        idx_b, _ = manual_step(d, [tuple(g) for g in B], ks, params, eta, 0.0, mu, keep={})
        torch.cuda.synchronize()
        for gi in range(len(groups)):
            assert torch.equal(idx_a[gi], idx_b[gi]), ("idx", step, gi)
            assert torch.equal(A[gi][0].view(torch.int16), B[gi][0].view(torch.int16)), ("W", step, gi)
        if step == 0:
            idx1 = [t.clone() for t in idx_a]
            # deferred: M still owes the decay; from M0 = 0 it equals G exactly
            for gi in range(len(groups)):
                assert torch.equal(A[gi][1].view(torch.int16), G1[gi].view(torch.int16)), ("M1", gi)
        print(f"# step {step}: idx and W bit-exact (benchmarked call vs entry points), every matrix",
              file=sys.stderr, flush=True)
    plan.flush_decay(mu)
    torch.cuda.synchronize()
    for gi in range(len(groups)):
        assert torch.equal(A[gi][1].view(torch.int16), B[gi][1].view(torch.int16)), ("M2", gi)

    # the oracle on every matrix: selections of both steps and the final
    # momentum, 32 matrices at a time (host copies of G1, G2 and M per batch)
    del B
    todo = [(gi, j) for gi, (_, _, b) in enumerate(groups) for j in range(b)]
    bad, done = [], 0
    with P.pool() as pool:
        for s0 in range(0, len(todo), 32):
            tasks = []
            for gi, j in todo[s0:s0 + 32]:
                r, c, _ = groups[gi]
                canon = (lambda x: x) if r <= c else (lambda x: np.ascontiguousarray(x.T))
                tasks.append(((gi, j), canon(_bits16(G1[gi][j])), canon(_bits16(A[gi][2][j])),
                              canon(_bits16(A[gi][1][j])), idx1[gi][j].cpu().numpy().astype(np.int64),
                              idx_a[gi][j].cpu().numpy().astype(np.int64), ks[gi], mu))
            for key, what in pool.imap_unordered(P.check_two_steps, tasks, chunksize=1):
                done += 1
                if what is not None:
                    bad.append((key, what))
            del tasks
            print(f"# oracle checked {done} of {len(todo)} matrices", file=sys.stderr, flush=True)
    assert not bad, bad[:10]
    print(f"# oracle: idx of both steps and M bit-exact on all {len(todo)} matrices", file=sys.stderr)


@pytest.mark.timeout(600)
def test_7b_normuon_benchmarked_call(d):
    """The NorMuon flavour of the benchmarked call (bench.py --flavor normuon:
    dion3_step_normuon, deferred) over the whole 7B set at f = 1/4: indices,
    W and the second moments V bit for bit against the entry points on every
    matrix (M once the pending decay is completed), and the first matrix of
    every group against the oracle ("Dion3: Full-Stack Orthogonal Updates",
    Section 2 for NorMuon's row normalisation and Frobenius rescale, Section 6
    for the flavour of the update)."""
    import oracle as O
    from helpers import bits, np_bits, rel_fro, to64
    from test_gpu_normuon import _manual_normuon, oracle_factors

    groups = synth.shape_groups("7b")
    f, mu, beta2, eps = 0.25, 0.95, 0.95, 1e-8
    eta = 0.02 / math.sqrt(f)
    ks = [d.dion3_k_from_fraction(min(r, c), f) for r, c, _ in groups]
    params = d.make_ns_params(ns_dtype=d.F16)
    A, B = [], []
    for gi, (r, c, b) in enumerate(groups):
        W = synth.weights(r, c, b, dtype="bf16", device=DEV, group_seed=gi)
        G = synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=gi, step=0)
        A.append([W, torch.zeros_like(W), G])
        B.append([W.clone(), torch.zeros_like(W), G.clone()])
    VA = [torch.zeros(b, min(r, c), dtype=torch.float32, device=DEV) for r, c, b in groups]
    VB = [v.clone() for v in VA]
    idx_a = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(groups, ks)]
    plan = d.StepPlan([g[0] for g in A], [g[1] for g in A], [g[2] for g in A], ks, idx_a, params)
    host = {gi: (to64(B[gi][0][0]), to64(B[gi][2][0])) for gi in range(len(groups))}
    plan.step_normuon(VA, eta, 0.0, mu, beta2, eps, deferred=True, has_prev=False)
    res = _manual_normuon(d, B, VB, ks, params, eta, mu, beta2, eps)
    plan.flush_decay(mu)
    torch.cuda.synchronize()
    for gi, (r, c, b) in enumerate(groups):
        idx_b, Og, rs = res[gi]
        assert torch.equal(idx_a[gi], idx_b), gi
        assert torch.equal(A[gi][0].view(torch.int16), B[gi][0].view(torch.int16)), ("W", gi)
        assert torch.equal(A[gi][1].view(torch.int16), B[gi][1].view(torch.int16)), ("M", gi)
        assert torch.equal(VA[gi], VB[gi]), ("V", gi)
        # the oracle on the group's first matrix (M0 = 0, V0 = 0)
        Wh, Gh = host[gi]
        out = O.dion3_step(Wh, np.zeros_like(Gh), Gh, k=ks[gi], mu=mu, eta=eta, fmt="bf16",
                           V=np.zeros(min(r, c)), beta2=beta2, nm_eps=eps)
        ij = idx_b[0].cpu().numpy()
        assert np.array_equal(ij, out["idx"]), gi
        assert np.array_equal(bits(B[gi][1][0]), np_bits(out["M"], torch.bfloat16)), gi
        Oc = to64(Og[0])
        err = rel_fro(Oc, out["O"])
        assert err <= 3e-2, (gi, err)
        fo, vn = oracle_factors(Oc, np.zeros(ks[gi]), beta2, eps)
        fg = rs[0].cpu().numpy()
        assert np.max(np.abs(fg - fo) / fo) <= 1e-5, gi
        assert np.max(np.abs(VB[gi][0].cpu().numpy()[ij] - vn) / vn) <= 1e-6, gi
        ax = 0 if r <= c else 1
        Gc = Gh if ax == 0 else Gh.T
        Wc = Wh if ax == 0 else Wh.T
        Uh = O.round_to(Oc * fg.astype(np.float64)[:, None], "f32")
        Wg, _ = O.apply_rows(Wc, Gc, ij, Uh, eta, 0.0, mu, "bf16")
        assert np.array_equal(bits(B[gi][0][0]), np_bits(Wg if ax == 0 else Wg.T, torch.bfloat16)), gi
        print(f"# normuon 7b group {gi}: O rel err {err:.3e}, every matrix bit-exact vs entry points",
              file=sys.stderr, flush=True)
