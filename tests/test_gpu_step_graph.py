"""The deferred step as HIP graphs built node by node (no stream capture;
"Dion3: Full-Stack Orthogonal Updates", Section 6: the step's launches have
the same dependencies every step, so recorded graphs are replayed per step),
in both forms: per-stream segments replayed on the library's streams, and
one graph of the whole step; the Muon and the NorMuon flavour.

A graph is created once over one set of tensors and replayed several times;
between replays new gradients are copied in and the same step runs eagerly on
a copy, with synchronisations around every replay.  After every replay the
selected indices, W and M (which both owe the same pending decay) must equal
the eager step's bit for bit."""

import math

import pytest
import torch

from muon_momentum_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def d():
    import muon_momentum_amd.dion3 as mod
    return mod


def _state(shapes, ks, seed0=0):
    Ws, Ms, Gs, ids = [], [], [], []
    for gi, (r, c, b) in enumerate(shapes):
        Ws.append(synth.weights(r, c, b, dtype="bf16", device=DEV, group_seed=seed0 + gi))
        Gs.append(synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=seed0 + gi, step=0))
        Ms.append(torch.zeros(b, r, c, dtype=Ws[-1].dtype, device=DEV))
        ids.append(torch.empty(b, ks[gi], dtype=torch.int32, device=DEV))
    return Ws, Ms, Gs, ids


def _replays_match(d, shapes, f, replays, seed0=0, one=False, normuon=False, wd=0.0):
    ks = [d.dion3_k_from_fraction(min(r, c), f) for r, c, _ in shapes]
    mu, eta = 0.95, 0.02 / math.sqrt(f)
    params = d.make_ns_params(ns_dtype=d.F16)
    A = _state(shapes, ks, seed0)
    B = [[t.clone() for t in ts] for ts in A]
    pa = d.StepPlan(A[0], A[1], A[2], ks, A[3], params)
    pb = d.StepPlan(B[0], B[1], B[2], ks, B[3], params)
    # NorMuon: second moments per line of the selection axis, one state per copy
    Va = [torch.zeros(b, min(r, c), dtype=torch.float32, device=DEV) for r, c, b in shapes]
    Vb = [v.clone() for v in Va]

    def eager(has_prev):
        if normuon:
            pa.step_normuon(Va, eta, wd, mu, deferred=True, has_prev=has_prev)
        else:
            pa.step_deferred(eta, wd, mu, has_prev=has_prev)

    eager(False)
    if normuon:
        pb.step_normuon(Vb, eta, wd, mu, deferred=True, has_prev=False)
    else:
        pb.step_deferred(eta, wd, mu, has_prev=False)
    torch.cuda.synchronize()
    if normuon:
        graph = pb.graph_normuon(Vb, eta, wd, mu, has_prev=True, one=one)
    else:
        graph = pb.graph(eta, wd, mu, has_prev=True, one=one)
    torch.cuda.synchronize()
    for step in range(1, replays + 1):
        for gi, (r, c, b) in enumerate(shapes):
            Gn = synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=seed0 + gi, step=step)
            A[2][gi].copy_(Gn)
            B[2][gi].copy_(Gn)
            del Gn
        torch.cuda.synchronize()
        eager(True)
        torch.cuda.synchronize()
        graph.launch()
        torch.cuda.synchronize()
        for gi in range(len(shapes)):
            assert torch.equal(A[3][gi], B[3][gi]), ("idx", step, gi)
            assert torch.equal(A[0][gi].view(torch.int16), B[0][gi].view(torch.int16)), ("W", step, gi)
            assert torch.equal(A[1][gi].view(torch.int16), B[1][gi].view(torch.int16)), ("M", step, gi)
            if normuon:
                assert torch.equal(Va[gi].view(torch.int32), Vb[gi].view(torch.int32)), ("V", step, gi)
    graph.destroy()
    torch.cuda.synchronize()


@pytest.mark.parametrize("one", [False, True])
@pytest.mark.parametrize("f", [0.25, 1.0])
def test_step_graph_replays_match_eager(d, f, one):
    # three (k, m) classes (rows and columns selected together), a square class
    # at f = 1, and 256 x 256 tiles (the 1024-row groups); the segmented and
    # the single-graph form
    _replays_match(d, [(256, 1024, 6), (1024, 256, 3), (512, 512, 2), (1024, 2048, 2)], f, replays=4, one=one)


@pytest.mark.parametrize("normuon", [False, True])
def test_step_graph_with_weight_decay(d, normuon):
    """Weight decay on: the graph also holds the decay of the lines the update
    does not touch (a kernel of its own after a fused update)."""
    _replays_match(d, [(256, 1024, 4), (1024, 256, 2), (1024, 2048, 2)], 0.25, replays=3, normuon=normuon,
                   wd=0.01)


@pytest.mark.parametrize("one", [False, True])
def test_normuon_step_graph_replays_match_eager(d, one):
    """The deferred NorMuon step as graphs (dion3_step_normuon_graph_create):
    idx, W, M and the second moments V bit-exact after every replay."""
    _replays_match(d, [(256, 1024, 6), (1024, 256, 3), (512, 512, 2), (1024, 2048, 2)], 0.25, replays=3,
                   one=one, normuon=True)


@pytest.mark.parametrize("one", [False, True])
@pytest.mark.timeout(600)
def test_step_graph_7b_matches_eager(d, one):
    """The benchmarked workload: 7B shape set, f = 1/4, two replays."""
    _replays_match(d, synth.shape_groups("7b"), 0.25, replays=2, seed0=0, one=one)


@pytest.mark.timeout(600)
def test_normuon_step_graph_7b_matches_eager(d):
    """The NorMuon flavour of the benchmarked workload as segmented graphs:
    7B shape set, f = 1/4, two replays, V bit-exact as well."""
    _replays_match(d, synth.shape_groups("7b"), 0.25, replays=2, seed0=0, normuon=True)


def test_step_graph_after_release(d):
    """dion3_release destroys the library's streams: a segmented graph built
    on them then refuses to launch (DION3_ERR_INVALID_ARG, nothing enqueued),
    while the single-graph form, which uses no library stream, still runs;
    the next eager step recreates the streams."""
    shapes = [(256, 1024, 2)]
    ks = [d.dion3_k_from_fraction(256, 0.25)]
    params = d.make_ns_params(ns_dtype=d.F16)
    A = _state(shapes, ks)
    plan = d.StepPlan(A[0], A[1], A[2], ks, A[3], params)
    plan.step_deferred(0.04, 0.0, 0.95, has_prev=False)
    g_seg = plan.graph(0.04, 0.0, 0.95, has_prev=True)
    g_one = plan.graph(0.04, 0.0, 0.95, has_prev=True, one=True)
    torch.cuda.synchronize()
    assert d.lib.dion3_release() == 0
    with pytest.raises(d.Dion3Error, match=r"\(-1\)"):
        g_seg.launch()
    g_one.launch()
    torch.cuda.synchronize()
    plan.step_deferred(0.04, 0.0, 0.95, has_prev=True)
    torch.cuda.synchronize()
    g_seg.destroy()
    g_one.destroy()
