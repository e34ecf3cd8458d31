"""The whole step captured in a HIP graph and replayed ("Dion3: Full-Stack
Orthogonal Updates", Section 6: the launches of a step have the same
dependency structure every step, so a captured graph replaces them).

The step forks onto the library's own streams with events; capture follows
the fork and the join.  A captured deferred step (has_prev = 1) is replayed
several times, with new gradients copied in between replays and eager work and
synchronisation around every replay; after each replay idx, W and M must equal
those of the same step run eagerly on a copy, bit for bit."""

import pytest
import torch

from muon_momentum_amd import synth

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="graph capture of the multi-stream step crashed the host process inside "
                            "the runtime's end of capture on MI355X (twice: with the compute-unit-masked "
                            "stream in the capture, then with non-blocking streams only); the step now "
                            "refuses capture (DION3_ERR_UNSUPPORTED) until a cause is shown"),
]
DEV = "cuda"


@pytest.fixture(scope="module")
def d():
    import muon_momentum_amd.dion3 as mod
    return mod


def _state(shapes, ks, dt):
    Ws, Ms, Gs, ids = [], [], [], []
    for gi, (r, c, b) in enumerate(shapes):
        Ws.append(synth.weights(r, c, b, dtype=dt, device=DEV, group_seed=gi))
        Gs.append(synth.gradient(r, c, b, dtype=dt, device=DEV, group_seed=gi, step=0))
        Ms.append(torch.zeros(b, r, c, dtype=Ws[-1].dtype, device=DEV))
        ids.append(torch.empty(b, ks[gi], dtype=torch.int32, device=DEV))
    return Ws, Ms, Gs, ids


@pytest.mark.parametrize("f", [0.25, 1.0])
def test_graph_replay_matches_eager(d, f):
    # two (k, m) classes (rows and columns selected together), a square class
    # at f = 1, and the 256 x 256 tiles (the 1024-row groups)
    shapes = [(256, 1024, 6), (1024, 256, 3), (512, 512, 2), (1024, 2048, 2)]
    ks = [d.dion3_k_from_fraction(min(r, c), f) for r, c, _ in shapes]
    mu, eta = 0.95, 0.02 / f ** 0.5
    params = d.make_ns_params(ns_dtype=d.F16)
    A = _state(shapes, ks, "bf16")
    B = [[t.clone() for t in ts] for ts in A]
    pa = d.StepPlan(A[0], A[1], A[2], ks, A[3], params)
    pb = d.StepPlan(B[0], B[1], B[2], ks, B[3], params)
    # first step eagerly on both (no pending decay yet)
    pa.step_deferred(eta, 0.0, mu, has_prev=False)
    pb.step_deferred(eta, 0.0, mu, has_prev=False)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            pb.step_deferred(eta, 0.0, mu, has_prev=True)
    torch.cuda.synchronize()

    for step in range(1, 5):
        for gi, (r, c, b) in enumerate(shapes):
            Gn = synth.gradient(r, c, b, dtype="bf16", device=DEV, group_seed=gi, step=step)
            A[2][gi].copy_(Gn)
            B[2][gi].copy_(Gn)
        torch.cuda.synchronize()
        pa.step_deferred(eta, 0.0, mu, has_prev=True)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for gi in range(len(shapes)):
            assert torch.equal(A[3][gi], B[3][gi]), ("idx", step, gi)
            assert torch.equal(A[0][gi].view(torch.int16), B[0][gi].view(torch.int16)), ("W", step, gi)
            assert torch.equal(A[1][gi].view(torch.int16), B[1][gi].view(torch.int16)), ("M", step, gi)
    del graph
    torch.cuda.synchronize()
