"""CPU checks of the C ABI: the library loads, exports every declared symbol,
computes its host-side helpers correctly and rejects invalid arguments before
launching anything (none of these calls reaches the GPU)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dion3.h")

d = pytest.importorskip("muon_momentum_amd.dion3")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dion3_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared()
    assert len(names) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", d.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(dion3_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(d.lib, n)


def test_k_from_fraction_matches_oracle():
    rng = np.random.default_rng(1)
    cases = [(10, 0.25), (4096, 0.25), (2048, 0.125), (10, 0.7), (3, 1 / 3), (1, 1.0), (5120, 0.25),
             (1000, 1e-12), (7, 0.1 * 3)]
    cases += [(int(rng.integers(1, 40000)), float(rng.random()) or 0.5) for _ in range(2000)]
    for n, f in cases:
        assert d.dion3_k_from_fraction(n, f) == O.k_from_fraction(n, f), (n, f)
    for n, f in [(0, 0.5), (10, 0.0), (10, 1.0000001), (10, float("nan")), (-1, 0.5)]:
        assert d.lib.dion3_k_from_fraction(n, f) == -1


def test_canonical_orientation():
    for (r, c, ax, want) in [(4096, 4096, -1, (4096, 4096, 0)), (4096, 11008, -1, (4096, 11008, 0)),
                             (11008, 4096, -1, (4096, 11008, 1)), (256, 1024, 1, (1024, 256, 1)),
                             (300, 200, 0, (300, 200, 0))]:
        g = d.Group(r, c, 2, r * c, d.BF16, ax)
        assert d.dion3_canonical(g) == want
        assert O.canonical_axis(r, c, ax) == want[2]
    with pytest.raises(d.Dion3Error):
        d.dion3_canonical(d.Group(0, 5, 1, 0, d.BF16, -1))
    with pytest.raises(d.Dion3Error):
        d.dion3_canonical(d.Group(5, 5, 2, 24, d.BF16, -1))   # stride < rows*cols


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def test_invalid_arguments_rejected_without_launch():
    L = d.lib
    g = d.Group(64, 128, 2, 64 * 128, d.BF16, -1)
    gp = ctypes.byref(g)
    need = L.dion3_rowsel_workspace_bytes(gp)
    assert need >= 256
    # k outside [1, n]
    assert L.dion3_momentum_rowsel(gp, FAKE, FAKE, 0, FAKE, None, None, FAKE, need, None) == -1
    assert L.dion3_momentum_rowsel(gp, FAKE, FAKE, 65, FAKE, None, None, FAKE, need, None) == -1
    # null tensors
    assert L.dion3_momentum_rowsel(gp, None, FAKE, 4, FAKE, None, None, FAKE, need, None) == -1
    # workspace too small
    assert L.dion3_momentum_rowsel(gp, FAKE, FAKE, 4, FAKE, None, None, FAKE, need - 1, None) == -3
    # unsupported storage dtype
    g16 = d.Group(64, 128, 2, 64 * 128, d.F16, -1)
    assert L.dion3_momentum_rowsel(ctypes.byref(g16), FAKE, FAKE, 4, FAKE, None, None, FAKE, need, None) == -1
    # n beyond the top-k limit
    big = d.Group(40000, 40000, 1, 40000 * 40000, d.BF16, -1)
    nb = L.dion3_rowsel_workspace_bytes(ctypes.byref(big))
    assert L.dion3_momentum_rowsel(ctypes.byref(big), FAKE, FAKE, 4, FAKE, None, None, FAKE, nb, None) == -2
    # gather / apply
    assert L.dion3_gather_rows(gp, FAKE, FAKE, 0, FAKE, 1e-7, d.F16, FAKE, None) == -1
    assert L.dion3_gather_rows(gp, FAKE, FAKE, 4, FAKE, 1e-7, d.BF16, FAKE, None) == -1
    assert L.dion3_apply_rows(gp, FAKE, FAKE, FAKE, 4, FAKE, d.BF16, 4 * 128, 0.1, 0.0, 0.9, None) == -1
    assert L.dion3_apply_rows(gp, FAKE, FAKE, FAKE, 4, FAKE, d.F16, 3 * 128, 0.1, 0.0, 0.9, None) == -1
    # symmetric building blocks: aliasing, sizes, dtypes, strides
    assert L.dion3_syrk(1, 64, 128, d.F16, FAKE, 0, FAKE, 0, 1.0, 0.0, None) == -1      # A == C
    assert L.dion3_syrk(2, 64, 128, d.F16, FAKE, 10, ctypes.c_void_p(0x2000), 4096, 1.0, 0.0, None) == -1
    assert L.dion3_syrk(1, 0, 128, d.F16, FAKE, 0, ctypes.c_void_p(0x2000), 0, 1.0, 0.0, None) == -1
    assert L.dion3_syrk(1, 64, 128, 7, FAKE, 0, ctypes.c_void_p(0x2000), 0, 1.0, 0.0, None) == -1
    assert L.dion3_sym_sq_add(1, 64, d.F16, FAKE, 0, FAKE, 0, FAKE, 0, 1.0, 1.0, 0.0, None) == -1
    assert L.dion3_sym_mul(1, 64, d.F16, FAKE, 0, ctypes.c_void_p(0x2000), 0, FAKE, 0, 1.0, None) == -1
    assert L.dion3_gemm(1, 64, 128, d.F16, FAKE, 0, ctypes.c_void_p(0x2000), 0, d.BF16,
                        ctypes.c_void_p(0x3000), 0, 1.0, None) == -1
    # gram_ns: k > m, bad params, workspace
    p = d.make_ns_params()
    pp = ctypes.byref(p)
    wsn = L.dion3_gram_ns_gathered_workspace_bytes(2, 64, 128, d.F16)
    assert wsn > 0
    assert L.dion3_gram_ns_gathered(2, 129, 128, pp, FAKE, ctypes.c_void_p(0x2000), FAKE, wsn, None) == -1
    assert L.dion3_gram_ns_gathered(2, 64, 128, pp, FAKE, ctypes.c_void_p(0x2000), FAKE, wsn - 1, None) == -3
    assert L.dion3_gram_ns_gathered(2, 64, 128, pp, FAKE, FAKE, FAKE, wsn, None) == -1          # X0 == O
    bad = d.make_ns_params(T=0, coeffs=[])
    assert L.dion3_gram_ns_gathered(2, 64, 128, ctypes.byref(bad), FAKE, ctypes.c_void_p(0x2000), FAKE, wsn, None) == -1
    # standard_ns: same argument checks
    wss = L.dion3_standard_ns_workspace_bytes(2, 64, 128, d.F16)
    assert wss > 0
    assert L.dion3_standard_ns(2, 129, 128, pp, FAKE, ctypes.c_void_p(0x2000), FAKE, wss, None) == -1
    assert L.dion3_standard_ns(2, 64, 128, pp, FAKE, ctypes.c_void_p(0x2000), FAKE, wss - 1, None) == -3
    assert L.dion3_standard_ns(2, 64, 128, pp, FAKE, FAKE, FAKE, wss, None) == -1        # X0 == O
    assert L.dion3_standard_ns(2, 64, 128, ctypes.byref(bad), FAKE, ctypes.c_void_p(0x2000), FAKE, wss,
                               None) == -1
    # whole step: workspace query and a too-small workspace
    groups = (d.Group * 2)(d.Group(64, 128, 2, 64 * 128, d.BF16, -1), d.Group(128, 64, 1, 128 * 64, d.BF16, -1))
    ks = (ctypes.c_int * 2)(16, 16)
    sw = L.dion3_step_workspace_bytes(2, groups, ks, pp)
    assert sw > 0
    ptrs = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert L.dion3_step(2, groups, ptrs, ptrs, ptrs, ks, ptrs, pp, 0.1, 0.0, 0.9, FAKE, sw - 1, None) == -3
    ks_bad = (ctypes.c_int * 2)(16, 65)
    assert L.dion3_step_workspace_bytes(2, groups, ks_bad, pp) == 0


def test_status_strings():
    for code in [0, -1, -2, -3, -4, 99]:
        assert isinstance(d.lib.dion3_status_string(code), bytes)


def test_gram_ns_gathered_workspace_formula():
    L = d.lib
    for (b, k, m, dt, es) in [(3, 100, 300, d.F16, 2), (1, 256, 1024, d.F32, 4)]:
        al = lambda v: (v + 255) // 256 * 256
        assert L.dion3_gram_ns_gathered_workspace_bytes(b, k, m, dt) == al(b * k * m * es) + 4 * al(b * k * k * es)


def test_standard_ns_workspace_formula():
    L = d.lib
    for (b, k, m, dt, es) in [(3, 100, 300, d.F16, 2), (1, 256, 1024, d.F32, 4)]:
        al = lambda v: (v + 255) // 256 * 256
        assert L.dion3_standard_ns_workspace_bytes(b, k, m, dt) == al(b * k * m * es) + 2 * al(b * k * k * es)


def test_normuon_entry_points_reject_invalid_arguments():
    """NorMuon scale, scaled update and NorMuon step: argument checks that fail
    before anything is launched (no GPU needed)."""
    L = d.lib
    g = d.Group(64, 300, 2, 64 * 300, d.BF16, -1)          # n = 64, m = 300
    gp = ctypes.byref(g)
    P2 = ctypes.c_void_p(0x2000)
    # normuon_scale: null pointers, k outside [1, n], beta2 outside [0, 1], eps < 0, dtype, stride
    assert L.dion3_normuon_scale(gp, None, 8, FAKE, d.F16, 8 * 300, P2, 0.95, 1e-8, P2, None) == -1
    assert L.dion3_normuon_scale(gp, FAKE, 8, FAKE, d.F16, 8 * 300, None, 0.95, 1e-8, P2, None) == -1
    assert L.dion3_normuon_scale(gp, FAKE, 8, FAKE, d.F16, 8 * 300, P2, 0.95, 1e-8, None, None) == -1
    assert L.dion3_normuon_scale(gp, FAKE, 0, FAKE, d.F16, 8 * 300, P2, 0.95, 1e-8, P2, None) == -1
    assert L.dion3_normuon_scale(gp, FAKE, 65, FAKE, d.F16, 65 * 300, P2, 0.95, 1e-8, P2, None) == -1
    assert L.dion3_normuon_scale(gp, FAKE, 8, FAKE, d.F16, 8 * 300, P2, 1.5, 1e-8, P2, None) == -1
    assert L.dion3_normuon_scale(gp, FAKE, 8, FAKE, d.F16, 8 * 300, P2, -0.1, 1e-8, P2, None) == -1
    assert L.dion3_normuon_scale(gp, FAKE, 8, FAKE, d.F16, 8 * 300, P2, 0.95, -1.0, P2, None) == -1
    assert L.dion3_normuon_scale(gp, FAKE, 8, FAKE, d.BF16, 8 * 300, P2, 0.95, 1e-8, P2, None) == -1
    assert L.dion3_normuon_scale(gp, FAKE, 8, FAKE, d.F16, 8 * 300 - 1, P2, 0.95, 1e-8, P2, None) == -1
    # apply_rows_scaled: null W / idx / O, k, stride, dtype pair
    assert L.dion3_apply_rows_scaled(gp, None, FAKE, FAKE, 8, FAKE, d.F16, 8 * 300, None, 0.1, 0.0, 0.9, None) == -1
    assert L.dion3_apply_rows_scaled(gp, FAKE, FAKE, None, 8, FAKE, d.F16, 8 * 300, None, 0.1, 0.0, 0.9, None) == -1
    assert L.dion3_apply_rows_scaled(gp, FAKE, FAKE, FAKE, 65, FAKE, d.F16, 65 * 300, None, 0.1, 0.0, 0.9,
                                     None) == -1
    assert L.dion3_apply_rows_scaled(gp, FAKE, FAKE, FAKE, 8, FAKE, d.F16, 100, None, 0.1, 0.0, 0.9, None) == -1
    assert L.dion3_apply_rows_scaled(gp, FAKE, FAKE, FAKE, 8, FAKE, d.BF16, 8 * 300, None, 0.1, 0.0, 0.9,
                                     None) == -1
    # step_normuon: V missing (array or one entry), beta2, workspace
    p = d.make_ns_params()
    pp = ctypes.byref(p)
    groups = (d.Group * 1)(g)
    ks = (ctypes.c_int * 1)(16)
    ptrs = (ctypes.c_void_p * 1)(0x1000)
    vs = (ctypes.c_void_p * 1)(0x3000)
    vnull = (ctypes.c_void_p * 1)(None)
    sw = L.dion3_step_workspace_bytes(1, groups, ks, pp)
    assert sw > 0
    args = (ptrs, ptrs, ptrs, ks, ptrs)
    assert L.dion3_step_normuon(1, groups, *args, None, 0, 0, pp, 0.1, 0.0, 0.9, 0.95, 1e-8, FAKE, sw, None) == -1
    assert L.dion3_step_normuon(1, groups, *args, vnull, 0, 0, pp, 0.1, 0.0, 0.9, 0.95, 1e-8, FAKE, sw, None) == -1
    assert L.dion3_step_normuon(1, groups, *args, vs, 0, 0, pp, 0.1, 0.0, 0.9, 2.0, 1e-8, FAKE, sw, None) == -1
    assert L.dion3_step_normuon(1, groups, *args, vs, 0, 0, pp, 0.1, 0.0, 0.9, 0.95, 1e-8, FAKE, sw - 1,
                                None) == -3


def test_group_gram_ns_workspace_and_argument_checks():
    """dion3_workspace_bytes serves both momentum_rowsel and the group form of
    dion3_gram_ns; the group form rejects invalid arguments before launching."""
    L = d.lib
    al = lambda v: (v + 255) // 256 * 256
    p = d.make_ns_params(ns_dtype=d.F16)
    pp = ctypes.byref(p)
    for (r, c, b, k) in [(64, 300, 3, 16), (500, 96, 2, 40), (128, 128, 1, 128)]:
        g = d.Group(r, c, b, r * c, d.BF16, -1)
        n, m = min(r, c), max(r, c)
        want = al(b * k * 8) + al(b * 8) + al(b * k * m * 2) + L.dion3_gram_ns_gathered_workspace_bytes(b, k, m, d.F16)
        assert L.dion3_gram_ns_workspace_bytes(ctypes.byref(g), k, pp) == want
        assert L.dion3_workspace_bytes(ctypes.byref(g), k, pp) == max(want, L.dion3_rowsel_workspace_bytes(ctypes.byref(g)))
    g = d.Group(64, 300, 2, 64 * 300, d.BF16, -1)
    gp = ctypes.byref(g)
    P2 = ctypes.c_void_p(0x2000)
    ws = L.dion3_gram_ns_workspace_bytes(gp, 16, pp)
    assert L.dion3_gram_ns_workspace_bytes(gp, 0, pp) == 0
    assert L.dion3_gram_ns_workspace_bytes(gp, 65, pp) == 0                     # k > n
    assert L.dion3_workspace_bytes(gp, 65, pp) == 0
    assert L.dion3_gram_ns(gp, None, FAKE, 16, pp, P2, FAKE, ws, None) == -1    # M missing
    assert L.dion3_gram_ns(gp, FAKE, None, 16, pp, P2, FAKE, ws, None) == -1    # idx missing
    assert L.dion3_gram_ns(gp, FAKE, FAKE, 16, pp, None, FAKE, ws, None) == -1  # O missing
    assert L.dion3_gram_ns(gp, FAKE, FAKE, 0, pp, P2, FAKE, ws, None) == -1
    assert L.dion3_gram_ns(gp, FAKE, FAKE, 16, pp, P2, FAKE, ws - 1, None) == -3
    assert L.dion3_gram_ns(gp, FAKE, FAKE, 16, pp, P2, None, ws, None) == -3
    bad = d.make_ns_params(T=0, coeffs=[])
    assert L.dion3_gram_ns(gp, FAKE, FAKE, 16, ctypes.byref(bad), P2, FAKE, ws, None) == -1
    g16 = d.Group(64, 300, 2, 64 * 300, d.F16, -1)                             # storage must be bf16 / f32
    assert L.dion3_gram_ns(ctypes.byref(g16), FAKE, FAKE, 16, pp, P2, FAKE, ws, None) == -1


def test_step_refuses_unsupported_type_pairs():
    """The gather and the update take fp16 or fp32 Newton-Schulz buffers and
    bf16 or fp32 storage; the whole-step calls and the group form of
    dion3_gram_ns refuse any other pair in their planning, before any launch
    (so no M or W is touched)."""
    L = d.lib
    ok = d.make_ns_params(ns_dtype=d.F16)
    b16 = d.make_ns_params(ns_dtype=d.BF16)
    groups = (d.Group * 2)(d.Group(64, 128, 2, 64 * 128, d.BF16, -1), d.Group(128, 64, 1, 128 * 64, d.BF16, -1))
    ks = (ctypes.c_int * 2)(16, 16)
    ptrs = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    sw = L.dion3_step_workspace_bytes(2, groups, ks, ctypes.byref(ok))
    assert sw > 0
    assert L.dion3_step_workspace_bytes(2, groups, ks, ctypes.byref(b16)) == 0
    f16_groups = (d.Group * 2)(d.Group(64, 128, 2, 64 * 128, d.F16, -1), d.Group(128, 64, 1, 128 * 64, d.BF16, -1))
    assert L.dion3_step_workspace_bytes(2, f16_groups, ks, ctypes.byref(ok)) == 0
    for gr, p in [(groups, b16), (f16_groups, ok)]:
        pp = ctypes.byref(p)
        assert L.dion3_step(2, gr, ptrs, ptrs, ptrs, ks, ptrs, pp, 0.1, 0.0, 0.9, FAKE, sw, None) == -1
        assert L.dion3_step_deferred(2, gr, ptrs, ptrs, ptrs, ks, ptrs, 1, pp, 0.1, 0.0, 0.9, FAKE, sw, None) == -1
        vs = (ctypes.c_void_p * 2)(0x3000, 0x4000)
        assert L.dion3_step_normuon(2, gr, ptrs, ptrs, ptrs, ks, ptrs, vs, 1, 1, pp, 0.1, 0.0, 0.9, 0.95, 1e-8,
                                    FAKE, sw, None) == -1
        out = ctypes.c_void_p()
        assert L.dion3_step_graph_create(2, gr, ptrs, ptrs, ptrs, ks, ptrs, 1, pp, 0.1, 0.0, 0.9, FAKE, sw, 0,
                                         ctypes.byref(out)) == -1
        assert out.value is None
        assert L.dion3_step_normuon_graph_create(2, gr, ptrs, ptrs, ptrs, ks, ptrs, vs, 1, pp, 0.1, 0.0, 0.9,
                                                 0.95, 1e-8, FAKE, sw, 0, ctypes.byref(out)) == -1
        assert out.value is None
    g = d.Group(64, 300, 2, 64 * 300, d.BF16, -1)
    ws = L.dion3_gram_ns_workspace_bytes(ctypes.byref(g), 16, ctypes.byref(b16))
    assert L.dion3_gram_ns(ctypes.byref(g), FAKE, FAKE, 16, ctypes.byref(b16), ctypes.c_void_p(0x2000), FAKE, ws,
                           None) == -1


def test_count_nonfinite_argument_checks():
    """The finite check validates before any launch: pointers, n and dtype."""
    L = d.lib
    assert L.dion3_count_nonfinite(None, d.F32, 10, FAKE, None) == -1
    assert L.dion3_count_nonfinite(FAKE, d.F32, 10, None, None) == -1
    assert L.dion3_count_nonfinite(FAKE, d.F32, 0, FAKE, None) == -1
    assert L.dion3_count_nonfinite(FAKE, 7, 10, FAKE, None) == -1


def test_release_without_gpu_work_is_a_no_op():
    """dion3_release frees only what the library created; with nothing created
    it makes no HIP call and succeeds (twice in a row as well)."""
    assert d.lib.dion3_release() == 0
    assert d.lib.dion3_release() == 0


def test_step_graph_argument_checks():
    """dion3_step_graph_create validates like the step before any HIP call;
    launching or destroying a missing graph is handled."""
    L = d.lib
    p = d.make_ns_params()
    pp = ctypes.byref(p)
    groups = (d.Group * 2)(d.Group(64, 128, 2, 64 * 128, d.BF16, -1), d.Group(128, 64, 1, 128 * 64, d.BF16, -1))
    ks = (ctypes.c_int * 2)(16, 16)
    ptrs = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    sw = L.dion3_step_workspace_bytes(2, groups, ks, pp)
    out = ctypes.c_void_p()
    args = (ptrs, ptrs, ptrs, ks, ptrs, 1, pp, 0.1, 0.0, 0.9)
    assert L.dion3_step_graph_create(2, groups, *args, FAKE, sw - 1, 0, ctypes.byref(out)) == -3
    assert L.dion3_step_graph_create(2, groups, *args, FAKE, sw, 0, None) == -1
    assert L.dion3_step_graph_create(2, groups, *args, FAKE, sw, 2, ctypes.byref(out)) == -1   # unknown flag
    bad = (ctypes.c_int * 2)(16, 65)
    assert L.dion3_step_graph_create(2, groups, ptrs, ptrs, ptrs, bad, ptrs, 1, pp, 0.1, 0.0, 0.9, FAKE, sw, 0,
                                     ctypes.byref(out)) == -1
    nulls = (ctypes.c_void_p * 2)(0x1000, None)
    assert L.dion3_step_graph_create(2, groups, nulls, ptrs, ptrs, ks, ptrs, 1, pp, 0.1, 0.0, 0.9, FAKE, sw, 0,
                                     ctypes.byref(out)) == -1
    assert out.value is None
    # the NorMuon form: the same checks, and the second-moment pointers
    vs = (ctypes.c_void_p * 2)(0x3000, 0x4000)
    nargs = (ptrs, ptrs, ptrs, ks, ptrs)
    tail = (1, pp, 0.1, 0.0, 0.9, 0.95, 1e-8)
    NG = L.dion3_step_normuon_graph_create
    assert NG(2, groups, *nargs, vs, *tail, FAKE, sw - 1, 0, ctypes.byref(out)) == -3
    assert NG(2, groups, *nargs, vs, *tail, FAKE, sw, 0, None) == -1
    assert NG(2, groups, *nargs, vs, *tail, FAKE, sw, 2, ctypes.byref(out)) == -1
    assert NG(2, groups, *nargs, None, *tail, FAKE, sw, 0, ctypes.byref(out)) == -1
    assert NG(2, groups, *nargs, (ctypes.c_void_p * 2)(0x3000, None), *tail, FAKE, sw, 0, ctypes.byref(out)) == -1
    assert out.value is None
    assert L.dion3_graph_launch(None, None) == -1
    assert L.dion3_graph_destroy(None) == 0
