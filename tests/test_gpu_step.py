"""GPU parity of whole optimizer steps against the oracle.

Small workload: one 256 x 1024 fp32 matrix, f = 1 (plain Muon through Gram
Newton-Schulz with the restart), mu = 0.95, eta = 0.02, T = 5.  Plus a bf16
multi-group step whose row- and column-selected groups share one
Newton-Schulz batch."""

import numpy as np
import pytest
import torch

import oracle as O
from helpers import bits, manual_step, np_bits, rel_fro, to64
from muon_momentum_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}


@pytest.fixture(scope="module")
def d():
    import muon_momentum_amd.dion3 as mod
    return mod


def test_config1_fp32_f1_three_steps(d):
    rows, cols, T = 256, 1024, 5
    mu, eta = 0.95, 0.02
    W = synth.weights(rows, cols, 1, dtype="f32", device=DEV)
    M = torch.zeros(1, rows, cols, dtype=torch.float32, device=DEV)
    Wr, Mr = to64(W)[0], to64(M)[0]
    params = d.make_ns_params(ns_dtype=d.F32)
    k = d.dion3_k_from_fraction(rows, 1.0)
    for step in range(3):
        G = synth.gradient(rows, cols, 1, dtype="f32", device=DEV, step=step)
        out = O.dion3_step(Wr, Mr, to64(G)[0], k=k, mu=mu, eta=eta, fmt="f32")
        Wg_before = to64(W)[0]
        idxs, Os = manual_step(d, [(W, M, G)], [k], params, eta, 0.0, mu)
        assert np.array_equal(idxs[0].cpu().numpy()[0], out["idx"])
        assert np.array_equal(bits(M[0]), np_bits(out["M"], torch.float32))       # M bit-exact
        Og = to64(Os[0])[0]
        err = rel_fro(Og, out["O"])
        assert err <= 1e-4, (step, err)
        # W: the oracle's fused rounding applied to the GPU's own O is bit-exact
        Wg_ref, _ = O.apply_rows(Wg_before, O.momentum_accumulate(Mr, to64(G)[0], "f32"), out["idx"], Og,
                                 eta, 0.0, mu, "f32")
        assert np.array_equal(bits(W[0]), np_bits(Wg_ref, torch.float32))
        Wr, Mr = out["W"], out["M"]
        # the GPU trajectory stays within tolerance of the oracle's
        assert rel_fro(to64(W)[0] - to64(synth.weights(rows, cols, 1, dtype="f32", device=DEV))[0],
                       Wr - to64(synth.weights(rows, cols, 1, dtype="f32", device=DEV))[0]) <= 1e-4


def _groups(shapes, dt, step, seed0=0):
    out = []
    for gi, (r, c, b) in enumerate(shapes):
        W = synth.weights(r, c, b, dtype=dt, device=DEV, group_seed=seed0 + gi)
        M = synth.gradient(r, c, b, dtype=dt, device=DEV, group_seed=seed0 + gi + 50, step=99) * 0.5
        M = M.to(TD[dt])
        G = synth.gradient(r, c, b, dtype=dt, device=DEV, group_seed=seed0 + gi, step=step)
        out.append((W, M, G))
    return out


@pytest.mark.parametrize("f", [0.25, 1.0])
def test_multigroup_bf16_step_matches_manual_and_oracle(d, f):
    shapes = [(128, 512, 3), (512, 128, 2), (256, 256, 2), (96, 200, 1)]
    dt = "bf16"
    mu, eta, wd = 0.95, 0.02 / f ** 0.5, 0.0
    params = d.make_ns_params(ns_dtype=d.F16)
    ks = [d.dion3_k_from_fraction(min(r, c), f) for r, c, _ in shapes]
    A = _groups(shapes, dt, step=0)
    B = [(W.clone(), M.clone(), G.clone()) for W, M, G in A]
    host = [(to64(W), to64(M), to64(G)) for W, M, G in A]
    # whole step in one call
    idx_a = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(shapes, ks)]
    d.dion3_step([g[0] for g in A], [g[1] for g in A], [g[2] for g in A], ks, idx_a, eta, wd, mu, params)
    # the same through the individual entry points
    idx_b, Os = manual_step(d, B, ks, params, eta, wd, mu)
    for gi in range(len(shapes)):
        assert np.array_equal(idx_a[gi].cpu().numpy(), idx_b[gi].cpu().numpy())
        assert np.array_equal(bits(A[gi][0]), bits(B[gi][0]))
        assert np.array_equal(bits(A[gi][1]), bits(B[gi][1]))
    # oracle, matrix by matrix
    for gi, (r, c, b) in enumerate(shapes):
        Wh, Mh, Gh = host[gi]
        for j in range(b):
            out = O.dion3_step(Wh[j], Mh[j], Gh[j], k=ks[gi], mu=mu, eta=eta, fmt=dt)
            assert np.array_equal(idx_b[gi].cpu().numpy()[j], out["idx"])
            assert np.array_equal(bits(B[gi][1][j]), np_bits(out["M"], torch.bfloat16))
            Og = to64(Os[gi][j])
            assert rel_fro(Og, out["O"]) <= 3e-2
            Mc = O.momentum_accumulate(Mh[j], Gh[j], dt)
            ax = O.canonical_axis(r, c)
            Wc, Mcc = (Wh[j], Mc) if ax == 0 else (Wh[j].T, Mc.T)
            Wg, _ = O.apply_rows(Wc, Mcc, out["idx"], Og, eta, wd, mu, dt)
            if ax == 1:
                Wg = Wg.T
            assert np.array_equal(bits(B[gi][0][j]), np_bits(Wg, torch.bfloat16))


@pytest.mark.parametrize("shapes", [
    [(256, 256, 2), (128, 512, 3), (512, 128, 2)],   # square matrices, then a class of two groups
    [(128, 512, 3)],                                 # a single class
    [(200, 96, 1), (128, 512, 1), (512, 128, 1)],    # single matrices, two of them in one class
    [(64, 256, 2), (128, 256, 1), (96, 320, 2), (256, 256, 1), (64, 512, 3)],   # five classes
    # the step takes classes in order of increasing momentum traffic: these
    # groups arrive in another order
    [(128, 512, 3), (512, 128, 2), (256, 256, 1)],
    [(64, 512, 3), (256, 256, 1), (96, 320, 2), (128, 256, 1), (64, 256, 2)],
])
def test_step_class_layouts_match_manual(d, shapes):
    """Classes made of several groups, a single class, classes of single
    matrices: the whole step equals the entry points run one class at a time."""
    dt = "bf16"
    mu, eta, wd = 0.95, 0.03, 0.01
    params = d.make_ns_params(ns_dtype=d.F16)
    ks = [d.dion3_k_from_fraction(min(r, c), 0.25) for r, c, _ in shapes]
    A = _groups(shapes, dt, step=2, seed0=20)
    B = [(W.clone(), M.clone(), G.clone()) for W, M, G in A]
    idx_a = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(shapes, ks)]
    d.dion3_step([g[0] for g in A], [g[1] for g in A], [g[2] for g in A], ks, idx_a, eta, wd, mu, params)
    idx_b, _ = manual_step(d, B, ks, params, eta, wd, mu)
    torch.cuda.synchronize()
    for gi in range(len(shapes)):
        assert np.array_equal(idx_a[gi].cpu().numpy(), idx_b[gi].cpu().numpy()), gi
        assert np.array_equal(bits(A[gi][0]), bits(B[gi][0])), ("W", gi)
        assert np.array_equal(bits(A[gi][1]), bits(B[gi][1])), ("M", gi)


def test_step_deterministic(d):
    shapes = [(256, 768, 2), (768, 256, 1)]
    ks = [64, 64]
    res = []
    for _ in range(2):
        A = _groups(shapes, "bf16", step=1, seed0=10)
        idx = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(shapes, ks)]
        d.dion3_step([g[0] for g in A], [g[1] for g in A], [g[2] for g in A], ks, idx, 0.04, 0.0, 0.95)
        torch.cuda.synchronize()
        res.append([bits(g[0]) for g in A] + [bits(g[1]) for g in A] + [i.cpu().numpy() for i in idx])
    for a, b in zip(*res):
        assert np.array_equal(a, b)


def test_deferred_decay_matches_immediate(d):
    """dion3_step_deferred over three steps reproduces dion3_step bit for bit:
    indices and W after every step, M once the pending decay is completed."""
    shapes = [(128, 512, 3), (512, 128, 2), (256, 256, 2)]
    dt, f = "bf16", 0.25
    mu, eta = 0.95, 0.04
    params = d.make_ns_params(ns_dtype=d.F16)
    ks = [d.dion3_k_from_fraction(min(r, c), f) for r, c, _ in shapes]
    A = _groups(shapes, dt, step=0, seed0=30)
    B = [(W.clone(), M.clone(), G.clone()) for W, M, G in A]
    idx_a = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(shapes, ks)]
    idx_b = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(shapes, ks)]
    pa = d.StepPlan([g[0] for g in A], [g[1] for g in A], [g[2] for g in A], ks, idx_a, params)
    pb = d.StepPlan([g[0] for g in B], [g[1] for g in B], [g[2] for g in B], ks, idx_b, params)
    for step in range(3):
        for gi, (r, c, b) in enumerate(shapes):
            Gn = synth.gradient(r, c, b, dtype=dt, device=DEV, group_seed=30 + gi, step=step + 1)
            A[gi][2].copy_(Gn)
            B[gi][2].copy_(Gn)
        pa.step(eta, 0.0, mu)
        pb.step_deferred(eta, 0.0, mu, has_prev=step > 0)
        torch.cuda.synchronize()
        for gi in range(len(shapes)):
            assert np.array_equal(idx_a[gi].cpu().numpy(), idx_b[gi].cpu().numpy()), (step, gi)
            assert np.array_equal(bits(A[gi][0]), bits(B[gi][0])), (step, gi)
            Mb = B[gi][1].clone()
            d.dion3_decay_rows(Mb, idx_b[gi], ks[gi], mu)
            torch.cuda.synchronize()
            assert np.array_equal(bits(A[gi][1]), bits(Mb)), (step, gi)


@pytest.mark.parametrize("f,wd", [(0.25, 0.0), (0.25, 0.1), (1.0, 0.05)])
def test_fused_update_matches_immediate(d, f, wd):
    """Shapes on which the deferred Muon step fuses the update into the last
    Q X product (row-selected bf16 groups, k and m multiples of 256, at least
    128 tiles): W, idx and M (once its decay is completed) equal dion3_step's
    unfused update bit for bit over three steps.  At f = 1/4 the row-selected
    group shares its Newton-Schulz class with a column-selected one (one fused
    and one plain segment); at f = 1 the square group runs standard
    Newton-Schulz with the fused last product."""
    shapes = [(1024, 4096, 8), (4096, 1024, 4)] if f < 1 else [(1024, 1024, 8), (512, 1024, 2)]
    dt, mu, eta = "bf16", 0.95, 0.02 / f ** 0.5
    params = d.make_ns_params(ns_dtype=d.F16)
    ks = [d.dion3_k_from_fraction(min(r, c), f) for r, c, _ in shapes]
    A = _groups(shapes, dt, step=0, seed0=80)
    B = [(W.clone(), M.clone(), G.clone()) for W, M, G in A]
    idx_a = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(shapes, ks)]
    idx_b = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(shapes, ks)]
    pa = d.StepPlan([g[0] for g in A], [g[1] for g in A], [g[2] for g in A], ks, idx_a, params)
    pb = d.StepPlan([g[0] for g in B], [g[1] for g in B], [g[2] for g in B], ks, idx_b, params)
    d.dion3_timing_enable(512)
    try:
        for step in range(3):
            for gi, (r, c, b) in enumerate(shapes):
                Gn = synth.gradient(r, c, b, dtype=dt, device=DEV, group_seed=80 + gi, step=step + 1)
                A[gi][2].copy_(Gn)
                B[gi][2].copy_(Gn)
            pa.step(eta, wd, mu)
            pb.step_deferred(eta, wd, mu, has_prev=step > 0)
            torch.cuda.synchronize()
            for gi in range(len(shapes)):
                assert np.array_equal(idx_a[gi].cpu().numpy(), idx_b[gi].cpu().numpy()), (step, gi)
                assert np.array_equal(bits(A[gi][0]), bits(B[gi][0])), (step, gi)
                Mb = B[gi][1].clone()
                d.dion3_decay_rows(Mb, idx_b[gi], ks[gi], mu)
                torch.cuda.synchronize()
                assert np.array_equal(bits(A[gi][1]), bits(Mb)), (step, gi)
        rep = d.dion3_timing_report()
    finally:
        d.dion3_timing_enable(0)
    # the deferred steps did fuse (one fused launch per step)
    assert rep.get("qx_apply", (0, 0.0))[0] == 3, rep


def test_fused_update_falls_back_on_unaligned_rows(d):
    """A row-selected group whose matrices are not 16-byte aligned (batch
    stride padded by 3 elements) cannot take the fused update: the deferred
    step runs the plain last product and the apply pass instead, and still
    equals dion3_step bit for bit."""
    r, c, b, f = 1024, 4096, 8, 0.25
    mu, eta = 0.95, 0.04
    stride = r * c + 3
    params = d.make_ns_params(ns_dtype=d.F16)
    k = d.dion3_k_from_fraction(r, f)

    def strided(t):
        buf = torch.zeros(b * stride, dtype=t.dtype, device=DEV)
        v = buf.as_strided((b, r, c), (stride, c, 1))
        v.copy_(t)
        return v

    (W0, M0, G0), = _groups([(r, c, b)], "bf16", step=0, seed0=120)
    A = [strided(W0), strided(M0), strided(G0)]
    B = [strided(W0), strided(M0), strided(G0)]
    idx_a = torch.empty(b, k, dtype=torch.int32, device=DEV)
    idx_b = torch.empty(b, k, dtype=torch.int32, device=DEV)
    pa = d.StepPlan([A[0]], [A[1]], [A[2]], [k], [idx_a], params)
    pb = d.StepPlan([B[0]], [B[1]], [B[2]], [k], [idx_b], params)
    d.dion3_timing_enable(256)
    try:
        for step in range(2):
            Gn = synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=120, step=step + 1)
            A[2].copy_(Gn)
            B[2].copy_(Gn)
            pa.step(eta, 0.0, mu)
            pb.step_deferred(eta, 0.0, mu, has_prev=step > 0)
            torch.cuda.synchronize()
            assert torch.equal(idx_a, idx_b), step
            assert np.array_equal(bits(A[0]), bits(B[0])), step
        rep = d.dion3_timing_report()
    finally:
        d.dion3_timing_enable(0)
    assert "qx_apply" not in rep, rep


def test_momentum_ef_against_oracle(d):
    """M <- round(round(mu M) + G) on the previous selection, round(M + G) elsewhere."""
    for rows, cols, axis in [(300, 1000, 0), (900, 260, 1)]:
        n = rows if axis == 0 else cols
        kp = n // 4
        M = synth.gradient(rows, cols, 2, dtype="bf16", device=DEV, group_seed=3, step=5)
        G = synth.gradient(rows, cols, 2, dtype="bf16", device=DEV, group_seed=4, step=6)
        rng = np.random.default_rng(rows)
        prev = np.stack([np.sort(rng.choice(n, kp, replace=False)) for _ in range(2)]).astype(np.int32)
        Mh, Gh = to64(M), to64(G)
        idx = torch.empty(2, kp, dtype=torch.int32, device=DEV)
        d.dion3_momentum_rowsel_ef(M, G, kp, idx, torch.from_numpy(prev).to(DEV), kp, 0.95)
        torch.cuda.synchronize()
        for b in range(2):
            Mc = Mh[b] if axis == 0 else Mh[b].T
            Gc = Gh[b] if axis == 0 else Gh[b].T
            dec = Mc.copy()
            dec[prev[b]] = O.round_to(O.f32(0.95) * Mc[prev[b]], "bf16")
            ref = O.momentum_accumulate(dec, Gc, "bf16")
            ref = ref if axis == 0 else ref.T
            assert np.array_equal(bits(M[b]), np_bits(ref, torch.bfloat16)), (rows, cols, b)


def test_zero_gradient_step_leaves_w(d):
    """A matrix whose momentum and gradient are zero: every key is 0, so the
    first k lines are selected (ties to the lower index), the selected
    submatrix is zero, O = 0 (the eps guard of the normalisation) and W is
    unchanged bit for bit; its batch neighbours are updated as usual."""
    shapes = [(128, 512, 3), (512, 128, 2)]
    ks = [32, 32]
    params = d.make_ns_params(ns_dtype=d.F16)
    A = _groups(shapes, "bf16", step=4, seed0=60)
    for W, M, G in A:
        M[1].zero_()
        G[1].zero_()
    W0 = [W.clone() for W, _, _ in A]
    idx = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(shapes, ks)]
    plan = d.StepPlan([g[0] for g in A], [g[1] for g in A], [g[2] for g in A], ks, idx, params)
    plan.step(0.04, 0.0, 0.95)
    torch.cuda.synchronize()
    for gi, (W, M, G) in enumerate(A):
        assert np.array_equal(idx[gi][1].cpu().numpy(), np.arange(ks[gi]))
        assert np.array_equal(bits(W[1]), bits(W0[gi][1])), gi
        assert torch.count_nonzero(M[1]).item() == 0
        assert not np.array_equal(bits(W[0]), bits(W0[gi][0])), gi


def test_resume_round_trip_matches_straight_run(d):
    """Checkpoint and resume: three deferred steps in a row equal one deferred
    step, completion of its pending decay, a host round trip of W and M (the
    whole optimizer state besides the step count), and two more deferred
    steps (the first with no pending decay).  Indices, W and, once the last
    decay is completed, M agree bit for bit."""
    shapes = [(128, 512, 3), (512, 128, 2), (256, 256, 2)]
    dt, mu, eta = "bf16", 0.95, 0.04
    params = d.make_ns_params(ns_dtype=d.F16)
    ks = [d.dion3_k_from_fraction(min(r, c), 0.25) for r, c, _ in shapes]
    A = _groups(shapes, dt, step=0, seed0=70)
    B = [(W.clone(), M.clone(), G.clone()) for W, M, G in A]
    idx_a = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(shapes, ks)]
    idx_b = [t.clone() for t in idx_a]
    pa = d.StepPlan([g[0] for g in A], [g[1] for g in A], [g[2] for g in A], ks, idx_a, params)
    pb = d.StepPlan([g[0] for g in B], [g[1] for g in B], [g[2] for g in B], ks, idx_b, params)

    def grads(step):
        for gi, (r, c, b) in enumerate(shapes):
            Gn = synth.gradient(r, c, b, dtype=dt, device=DEV, group_seed=70 + gi, step=step + 1)
            A[gi][2].copy_(Gn)
            B[gi][2].copy_(Gn)

    grads(0)
    pa.step_deferred(eta, 0.0, mu, has_prev=False)
    pb.step_deferred(eta, 0.0, mu, has_prev=False)
    # checkpoint of B: complete the pending decay, save W and M on the host,
    # scribble over the device state, restore it
    pb.flush_decay(mu)
    torch.cuda.synchronize()
    saved = [(W.cpu().clone(), M.cpu().clone()) for W, M, _ in B]
    for W, M, _ in B:
        W.fill_(float("nan"))
        M.fill_(float("nan"))
    for (W, M, _), (Ws, Ms) in zip(B, saved):
        W.copy_(Ws.to(DEV))
        M.copy_(Ms.to(DEV))
    for step in (1, 2):
        grads(step)
        pa.step_deferred(eta, 0.0, mu, has_prev=True)
        pb.step_deferred(eta, 0.0, mu, has_prev=step > 1)   # the restored M owes no decay
        torch.cuda.synchronize()
        for gi in range(len(shapes)):
            assert torch.equal(idx_a[gi], idx_b[gi]), (step, gi)
            assert np.array_equal(bits(A[gi][0]), bits(B[gi][0])), (step, gi)
    pa.flush_decay(mu)
    pb.flush_decay(mu)
    torch.cuda.synchronize()
    for gi in range(len(shapes)):
        assert np.array_equal(bits(A[gi][1]), bits(B[gi][1])), gi


def test_concurrent_callers_match_sequential(d):
    """Two host threads, each with its own stream and tensors, enqueue three
    deferred steps at the same time (the library's streams and events are
    shared under one lock): each thread's idx, W and M equal the same steps
    run alone, bit for bit."""
    import threading

    shapes = [(512, 2048, 3), (2048, 512, 2)]
    f, mu, eta = 0.25, 0.95, 0.04
    params = d.make_ns_params(ns_dtype=d.F16)
    ks = [d.dion3_k_from_fraction(min(r, c), f) for r, c, _ in shapes]

    def make(seed0):
        A = _groups(shapes, "bf16", step=0, seed0=seed0)
        idx = [torch.empty(b, k, dtype=torch.int32, device=DEV) for (_, _, b), k in zip(shapes, ks)]
        return A, idx

    def run(A, idx, seed0, stream, barrier=None):
        with torch.cuda.stream(stream):
            plan = d.StepPlan([g[0] for g in A], [g[1] for g in A], [g[2] for g in A], ks, idx, params)
            if barrier is not None:
                barrier.wait()
            for step in range(3):
                for gi, (r, c, b) in enumerate(shapes):
                    A[gi][2].copy_(synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=seed0 + gi,
                                                  step=step + 1))
                plan.step_deferred(eta, 0.0, mu, has_prev=step > 0)
            stream.synchronize()

    seeds = [140, 150]
    ref = []
    for sd in seeds:                                   # each caller alone
        A, idx = make(sd)
        run(A, idx, sd, torch.cuda.Stream())
        ref.append(([bits(g[0]) for g in A], [bits(g[1]) for g in A], [i.cpu().numpy() for i in idx]))
    got = [make(sd) for sd in seeds]
    barrier = threading.Barrier(2)
    errors = []

    def worker(j):
        try:
            run(got[j][0], got[j][1], seeds[j], torch.cuda.Stream(), barrier)
        except Exception as e:                         # reported below
            errors.append(e)

    th = [threading.Thread(target=worker, args=(j,)) for j in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for j in range(2):
        A, idx = got[j]
        for gi in range(len(shapes)):
            assert np.array_equal(bits(A[gi][0]), ref[j][0][gi]), (j, gi)
            assert np.array_equal(bits(A[gi][1]), ref[j][1][gi]), (j, gi)
            assert np.array_equal(idx[gi].cpu().numpy(), ref[j][2][gi]), (j, gi)
