"""NorMuon flavour on the GPU against the oracle ("Dion3: Full-Stack Orthogonal
Updates", Section 2 for NorMuon's row normalisation and Frobenius rescale,
Section 6 for the flavour of the Dion3 update; reading of the missing equation
as in the oracle).

The moments and row factors are fp32 on the GPU and fp64 in the oracle:
they are compared within 1e-6 / 1e-5 relative.  The weight update is compared
bit for bit against the oracle's fused-rounding update applied to the GPU's
own O and row factors (one fp32 product O * factor, as the kernel does)."""

import numpy as np
import pytest
import torch

import oracle as O
from helpers import bits, np_bits, rel_fro, to64
from muon_momentum_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def d():
    import muon_momentum_amd.dion3 as mod
    return mod


def oracle_factors(Oc, v_sel, beta2, eps):
    """Row factors f with O_hat = f O, and the new moments, from the oracle."""
    Oh, vn = O.normuon_scale(Oc, v_sel, beta2, eps)
    nO = np.linalg.norm(Oc, axis=1)
    f = np.where(nO > 0, np.linalg.norm(Oh, axis=1) / np.where(nO > 0, nO, 1.0), np.nan)
    return f, vn


@pytest.mark.parametrize("odt", ["f32", "f16"])
@pytest.mark.parametrize("rows,cols,b,k", [(64, 300, 3, 20), (500, 96, 2, 40), (128, 128, 1, 128)])
def test_normuon_scale_vs_oracle(d, odt, rows, cols, b, k):
    rng = np.random.default_rng(rows + cols + k)
    n, m = min(rows, cols), max(rows, cols)
    M = torch.zeros(b, rows, cols, dtype=torch.bfloat16, device=DEV)     # only describes the group
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(b)]).astype(np.int32)
    Oc = rng.standard_normal((b, k, m)) * np.exp(rng.standard_normal((b, k, 1)))
    Oc[0, 1] = 0.0                                                      # a zero row
    Od = torch.from_numpy(Oc).to(TD[odt]).to(DEV)
    V0 = np.abs(rng.standard_normal((b, n))).astype(np.float32)
    Vd = torch.from_numpy(V0).to(DEV)
    rs = torch.empty(b, k, dtype=torch.float32, device=DEV)
    beta2, eps = 0.9, 1e-8
    d.dion3_normuon_scale(M, torch.from_numpy(idx).to(DEV), k, Od, Vd, rs, beta2, eps)
    torch.cuda.synchronize()
    V1, f1, On = Vd.cpu().numpy(), rs.cpu().numpy(), to64(Od)
    for j in range(b):
        fo, vn = oracle_factors(On[j], V0[j][idx[j]].astype(np.float64), beta2, eps)
        sel = np.zeros(n, dtype=bool)
        sel[idx[j]] = True
        assert np.array_equal(V1[j][~sel], V0[j][~sel])                # untouched lines
        assert np.max(np.abs(V1[j][idx[j]] - vn) / vn) <= 1e-6
        ok = ~np.isnan(fo)
        assert np.max(np.abs(f1[j][ok] - fo[ok]) / fo[ok]) <= 1e-5


@pytest.mark.parametrize("rows,cols", [(64, 300), (500, 96)])
def test_apply_rows_scaled(d, rows, cols):
    rng = np.random.default_rng(7)
    b, k = 2, 24
    n, m = min(rows, cols), max(rows, cols)
    W = synth.weights(rows, cols, b, dtype="bf16", device=DEV, group_seed=3)
    M = synth.gradient(rows, cols, b, dtype="bf16", device=DEV, group_seed=3)
    W2, M2, W3, M3 = W.clone(), M.clone(), W.clone(), M.clone()
    idx = torch.from_numpy(np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(b)])
                           .astype(np.int32)).to(DEV)
    Od = torch.from_numpy(rng.standard_normal((b, k, m)) * 0.05).half().to(DEV)
    rs = torch.from_numpy(np.exp(rng.standard_normal((b, k))).astype(np.float32)).to(DEV)
    eta, wd, mu = 0.03, 0.1, 0.9
    Wh, Mh = to64(W), to64(M)
    d.dion3_apply_rows_scaled(W, M, idx, k, Od, rs, eta, wd, mu)
    # a NULL factor is exactly the plain update
    d.dion3_apply_rows_scaled(W2, M2, idx, k, Od, None, eta, wd, mu)
    d.dion3_apply_rows(W3, M3, idx, k, Od, eta, wd, mu)
    torch.cuda.synchronize()
    assert torch.equal(W2.view(torch.int16), W3.view(torch.int16))
    assert torch.equal(M2.view(torch.int16), M3.view(torch.int16))
    ax = O.canonical_axis(rows, cols)
    for j in range(b):
        Uh = O.round_to(to64(Od[j]) * rs[j].cpu().numpy().astype(np.float64)[:, None], "f32")
        Wc, Mc = (Wh[j], Mh[j]) if ax == 0 else (Wh[j].T, Mh[j].T)
        Wr, Mr = O.apply_rows(Wc, Mc, idx[j].cpu().numpy(), Uh, eta, wd, mu, "bf16")
        if ax == 1:
            Wr, Mr = Wr.T, Mr.T
        assert np.array_equal(bits(W[j]), np_bits(Wr, torch.bfloat16))
        assert np.array_equal(bits(M[j]), np_bits(Mr, torch.bfloat16))


def _groups(shapes, step):
    out = []
    for gi, (r, c, b) in enumerate(shapes):
        W = synth.weights(r, c, b, dtype="bf16", device=DEV, group_seed=40 + gi)
        G = synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=40 + gi, step=step)
        out.append([W, torch.zeros_like(W), G])
    return out


def _manual_normuon(d, groups, Vs, ks, params, eta, mu, beta2, eps):
    """The NorMuon step through the individual entry points, batched like the
    whole step; returns idx, O, row factors per group."""
    classes = {}
    for gi, (W, M, G) in enumerate(groups):
        n, m, ax = d.dion3_canonical(d.make_group(M))
        classes.setdefault((ks[gi], m), []).append(gi)
    res = [None] * len(groups)
    for (k, m), members in classes.items():
        nb = sum(groups[g][0].shape[0] for g in members)
        X = torch.empty(nb, k, m, dtype=torch.float16, device=DEV)
        Ob = torch.empty_like(X)
        off, idxs = 0, {}
        for g in members:
            W, M, G = groups[g]
            b = M.shape[0]
            idx = torch.empty(b, k, dtype=torch.int32, device=DEV)
            sqn = torch.empty(b, dtype=torch.float64, device=DEV)
            d.dion3_momentum_rowsel(M, G, k, idx, None, sqn)
            d.dion3_gather_rows(M, idx, k, sqn, X[off:off + b], eps=params.eps)
            idxs[g] = idx
            off += b
        if k == m:
            d.dion3_standard_ns(X, Ob, params)
        else:
            d.dion3_gram_ns_gathered(X, Ob, params)
        off = 0
        for g in members:
            W, M, G = groups[g]
            b = M.shape[0]
            rs = torch.empty(b, k, dtype=torch.float32, device=DEV)
            Og = Ob[off:off + b]
            d.dion3_normuon_scale(M, idxs[g], k, Og, Vs[g], rs, beta2, eps)
            d.dion3_apply_rows_scaled(W, M, idxs[g], k, Og, rs, eta, 0.0, mu)
            res[g] = (idxs[g], Og.clone(), rs)
            off += b
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("f", [0.25, 1.0])
def test_normuon_step_matches_entry_points_and_oracle(d, f):
    shapes = [(128, 512, 3), (512, 128, 2), (256, 256, 2)]
    ks = [d.dion3_k_from_fraction(min(r, c), f) for r, c, _ in shapes]
    mu, eta, beta2, eps = 0.95, 0.02 / f ** 0.5, 0.95, 1e-8
    params = d.make_ns_params(ns_dtype=d.F16)
    A, B = _groups(shapes, 0), _groups(shapes, 0)
    VA = [torch.zeros(b, min(r, c), dtype=torch.float32, device=DEV) for r, c, b in shapes]
    VB = [v.clone() for v in VA]
    idx_a = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(shapes, ks)]
    plan = d.StepPlan([g[0] for g in A], [g[1] for g in A], [g[2] for g in A], ks, idx_a, params)
    for step in range(2):
        if step:
            for gi, (r, c, b) in enumerate(shapes):
                Gn = synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=40 + gi, step=step)
                A[gi][2].copy_(Gn)
                B[gi][2].copy_(Gn)
        host = [(to64(W), to64(M), to64(G)) for W, M, G in B]
        Vpre = [v.cpu().numpy().astype(np.float64) for v in VB]
        plan.step_normuon(VA, eta, 0.0, mu, beta2, eps)
        res = _manual_normuon(d, B, VB, ks, params, eta, mu, beta2, eps)
        for gi, (r, c, b) in enumerate(shapes):
            idx_b, Og, rs = res[gi]
            assert torch.equal(idx_a[gi], idx_b), (step, gi)
            assert torch.equal(A[gi][0].view(torch.int16), B[gi][0].view(torch.int16)), (step, gi)
            assert torch.equal(A[gi][1].view(torch.int16), B[gi][1].view(torch.int16)), (step, gi)
            assert torch.equal(VA[gi], VB[gi]), (step, gi)
            Wh, Mh, Gh = host[gi]
            ax = O.canonical_axis(r, c)
            for j in range(b):
                out = O.dion3_step(Wh[j], Mh[j], Gh[j], k=ks[gi], mu=mu, eta=eta, fmt="bf16",
                                   V=Vpre[gi][j], beta2=beta2, nm_eps=eps)
                ij = idx_b[j].cpu().numpy()
                assert np.array_equal(ij, out["idx"])
                assert np.array_equal(bits(B[gi][1][j]), np_bits(out["M"], torch.bfloat16))
                Oc = to64(Og[j])
                assert rel_fro(Oc, out["O"]) <= 3e-2
                fo, vn = oracle_factors(Oc, Vpre[gi][j][ij], beta2, eps)
                fg = rs[j].cpu().numpy()
                assert np.max(np.abs(fg - fo) / fo) <= 1e-5
                assert np.max(np.abs(VB[gi][j].cpu().numpy()[ij] - vn) / vn) <= 1e-6
                Mc = O.momentum_accumulate(Mh[j], Gh[j], "bf16")
                Wc, Mcc = (Wh[j], Mc) if ax == 0 else (Wh[j].T, Mc.T)
                Uh = O.round_to(Oc * fg.astype(np.float64)[:, None], "f32")
                Wg, _ = O.apply_rows(Wc, Mcc, ij, Uh, eta, 0.0, mu, "bf16")
                if ax == 1:
                    Wg = Wg.T
                assert np.array_equal(bits(B[gi][0][j]), np_bits(Wg, torch.bfloat16)), (step, gi, j)


def test_normuon_deferred_matches_immediate(d):
    shapes = [(128, 512, 3), (512, 128, 2), (256, 1024, 2)]
    ks = [d.dion3_k_from_fraction(min(r, c), 0.25) for r, c, _ in shapes]
    mu, eta = 0.95, 0.04
    params = d.make_ns_params(ns_dtype=d.F16)
    A, B = _groups(shapes, 0), _groups(shapes, 0)
    VA = [torch.zeros(b, min(r, c), dtype=torch.float32, device=DEV) for r, c, b in shapes]
    VB = [v.clone() for v in VA]
    ia = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(shapes, ks)]
    ib = [t.clone() for t in ia]
    pa = d.StepPlan([g[0] for g in A], [g[1] for g in A], [g[2] for g in A], ks, ia, params)
    pb = d.StepPlan([g[0] for g in B], [g[1] for g in B], [g[2] for g in B], ks, ib, params)
    for step in range(3):
        if step:
            for gi, (r, c, b) in enumerate(shapes):
                Gn = synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=40 + gi, step=step)
                A[gi][2].copy_(Gn)
                B[gi][2].copy_(Gn)
        pa.step_normuon(VA, eta, 0.0, mu)
        pb.step_normuon(VB, eta, 0.0, mu, deferred=True, has_prev=step > 0)
        torch.cuda.synchronize()
        for gi in range(len(shapes)):
            assert torch.equal(ia[gi], ib[gi]), (step, gi)
            assert torch.equal(A[gi][0].view(torch.int16), B[gi][0].view(torch.int16)), (step, gi)
            assert torch.equal(VA[gi], VB[gi]), (step, gi)
    pb.flush_decay(mu)
    torch.cuda.synchronize()
    for gi in range(len(shapes)):
        assert torch.equal(A[gi][1].view(torch.int16), B[gi][1].view(torch.int16)), gi
