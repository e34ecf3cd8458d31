"""Parity at the full sizes of the transformer shape sets, in the launch
configuration the benchmark times (same groups, same batched Newton-Schulz
classes, same kernels and grids).

The oracle runs the whole step on sampled matrices of every group: selected
indices and M bit for bit, the W update bit for bit given the GPU's
Newton-Schulz output O, and O within the fp16 tolerance (3e-2 relative
Frobenius), printed next to the extreme singular values of the normalised
input.  On the first step every eighth matrix of every group is also checked
against the oracle's selection from exact l1 norms of the step's momentum
(M0 = 0, so that momentum is G)."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from helpers import bits, manual_step, np_bits, rel_fro, to64
from muon_momentum_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def d():
    import muon_momentum_amd.dion3 as mod
    return mod


def check_selection(Mc, idx, k):
    """idx equals the oracle's selection from the exact l1 norms of Mc."""
    from oracle_pool import exact_l1
    assert np.array_equal(idx, O.select_rows(exact_l1(Mc), k))


def run_set(d, name, f, steps, sample, prop_every=8):
    groups = synth.shape_groups(name)
    tensors = []
    for gi, (r, c, b) in enumerate(groups):
        W = synth.weights(r, c, b, dtype="bf16", device=DEV, group_seed=gi)
        G = synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=gi, step=0)
        M = torch.zeros(b, r, c, dtype=torch.bfloat16, device=DEV)
        tensors.append([W, M, G])
    ks = [d.dion3_k_from_fraction(min(r, c), f) for r, c, _ in groups]
    eta, mu = 0.02 / math.sqrt(f), 0.95
    params = d.make_ns_params(ns_dtype=d.F16)
    # the oracle's state of every sampled matrix (W, M), followed across steps
    state = {(gi, j): [to64(tensors[gi][0][j]), np.zeros(groups[gi][:2])]
             for gi, js in sample.items() for j in js}
    worst = 0.0
    for step in range(steps):
        if step > 0:
            for gi, (r, c, b) in enumerate(groups):
                tensors[gi][2] = synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=gi, step=step)
        Gh = {key: to64(tensors[key[0]][2][key[1]]) for key in state}
        Wpre = {key: to64(tensors[key[0]][0][key[1]]) for key in state}
        idxs, Os = manual_step(d, [tuple(t) for t in tensors], ks, params, eta, 0.0, mu, keep=sample)
        for gi, (r, c, b) in enumerate(groups):
            ax = 0 if r <= c else 1
            idx_all = idxs[gi].cpu().numpy()
            if step == 0:
                for j in range(0, b, prop_every):
                    Gc = to64(tensors[gi][2][j])
                    check_selection(Gc if ax == 0 else Gc.T, idx_all[j], ks[gi])
            for j in sample.get(gi, []):
                Wh, Mh = state[(gi, j)]
                out = O.dion3_step(Wh, Mh, Gh[(gi, j)], k=ks[gi], mu=mu, eta=eta, fmt="bf16")
                where = (name, f, step, gi, j)
                assert np.array_equal(idx_all[j], out["idx"]), where
                assert np.array_equal(bits(tensors[gi][1][j]), np_bits(out["M"], torch.bfloat16)), where
                Og = to64(Os[gi][j])
                err = rel_fro(Og, out["O"])
                Mc = O.momentum_accumulate(Mh, Gh[(gi, j)], "bf16")
                # conditioning of the Newton-Schulz input next to every error figure
                X0 = O.frobenius_normalize((Mc if ax == 0 else Mc.T)[out["idx"]])
                sv = np.linalg.svd(X0, compute_uv=False)
                print(f"# {where}: O rel err {err:.3e}, X0 sigma_min {sv[-1]:.3e} sigma_max {sv[0]:.3e} "
                      f"(ratio {sv[-1] / sv[0]:.3e})", flush=True)
                worst = max(worst, err)
                assert err <= 3e-2, (where, err)
                Wc, Mcc = (Wpre[(gi, j)], Mc) if ax == 0 else (Wpre[(gi, j)].T, Mc.T)
                Wg, _ = O.apply_rows(Wc, Mcc, out["idx"], Og, eta, 0.0, mu, "bf16")
                if ax == 1:
                    Wg = Wg.T
                assert np.array_equal(bits(tensors[gi][0][j]), np_bits(Wg, torch.bfloat16)), where
                state[(gi, j)] = [out["W"], out["M"]]
        del Os
    del tensors
    torch.cuda.empty_cache()
    return worst


def test_7b_quarter(d):
    """The benchmarked workload: 7B shape set, f = 1/4, two matrices per group."""
    groups = synth.shape_groups("7b")
    worst = run_set(d, "7b", 0.25, 1, {gi: [0, b - 1] for gi, (_, _, b) in enumerate(groups)})
    print(f"7b f=1/4 worst O error {worst:.2e}")


def test_1b_eighth(d):
    groups = synth.shape_groups("1b")
    worst = run_set(d, "1b", 0.125, 1, {gi: [0, b - 1] for gi, (_, _, b) in enumerate(groups)})
    print(f"1b f=1/8 worst O error {worst:.2e}")


@pytest.mark.parametrize("f", [0.5, 1.0])
def test_7b_half_and_full(d, f):
    """f = 1/2 and f = 1 (plain Muon through Gram Newton-Schulz); the oracle
    follows one attention matrix, the property check covers every group."""
    worst = run_set(d, "7b", f, 1, {0: [0]})
    print(f"7b f={f} worst O error {worst:.2e}")


def test_14b_three_steps(d):
    """Three consecutive steps: the error-feedback momentum carries across and
    stays bit-exact; one square and one column-selected matrix followed."""
    groups = synth.shape_groups("14b")
    worst = run_set(d, "14b", 0.25, 3, {0: [0], 2: [groups[2][2] - 1]})
    print(f"14b f=1/4 three steps worst O error {worst:.2e}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,f,steps", [("7b", 0.25, 2), ("14b", 0.25, 3), ("7b", 0.5, 2), ("7b", 1.0, 1),
                                          ("1b", 0.125, 2)])
def test_deferred_matches_immediate_full(d, name, f, steps):
    """The benchmark's deferred step (decay carried into the next momentum
    pass, the update of row-selected groups fused into the last product) at
    the full size of every shape set against the immediate step with the
    separate update: indices and W bit for bit after each step, M bit for bit
    once the pending decay is completed."""
    groups = synth.shape_groups(name)
    ks = [d.dion3_k_from_fraction(min(r, c), f) for r, c, _ in groups]
    mu, eta = 0.95, 0.02 / math.sqrt(f)
    params = d.make_ns_params(ns_dtype=d.F16)
    sets = []
    for _ in range(2):
        Ws, Ms, Gs, ids = [], [], [], []
        for gi, (r, c, b) in enumerate(groups):
            Ws.append(synth.weights(r, c, b, dtype="bf16", device=DEV, group_seed=gi))
            Gs.append(synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=gi, step=0))
            Ms.append(torch.zeros(b, r, c, dtype=torch.bfloat16, device=DEV))
            ids.append(torch.empty(b, ks[gi], dtype=torch.int32, device=DEV))
        sets.append((Ws, Ms, Gs, ids, d.StepPlan(Ws, Ms, Gs, ks, ids, params)))
    (Wa, Ma, Ga, ia, pa), (Wb, Mb, Gb, ib, pb) = sets
    for step in range(steps):
        if step:
            for gi, (r, c, b) in enumerate(groups):
                Gn = synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=gi, step=step)
                Ga[gi].copy_(Gn)
                Gb[gi].copy_(Gn)
                del Gn
        pa.step(eta, 0.0, mu)
        pb.step_deferred(eta, 0.0, mu, has_prev=step > 0)
        torch.cuda.synchronize()
        for gi in range(len(groups)):
            assert torch.equal(ia[gi], ib[gi]), (name, f, step, gi)
            assert torch.equal(Wa[gi].view(torch.int16), Wb[gi].view(torch.int16)), (name, f, step, gi)
    pb.flush_decay(mu)
    torch.cuda.synchronize()
    for gi in range(len(groups)):
        assert torch.equal(Ma[gi].view(torch.int16), Mb[gi].view(torch.int16)), (name, f, gi)
    del sets, Wa, Ma, Ga, Wb, Mb, Gb, pa, pb
    torch.cuda.empty_cache()
    torch.cuda.empty_cache()
