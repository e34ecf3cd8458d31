"""Pins for the CPU oracle: each checks it against something other than itself
(closed forms, the pages' printed numbers, exact rational arithmetic, brute
force), chosen so that a plausible slip (a dropped term, a wrong sign or index,
a transposed operand) fails at least one of them."""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SHAPES = [(4, 4), (7, 19), (8, 32), (16, 64), (32, 128)]


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def sample(n, m, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, m)) * np.exp(rng.standard_normal((n, 1)))


# ---------------------------------------------------------------- Newton-Schulz
@pytest.mark.parametrize("n,m", SHAPES)
@pytest.mark.parametrize("restart", [(), (2,), (1, 3), (2, 4)])
def test_gram_equals_standard(n, m, restart):
    """Gram NS is standard NS rewritten; a restart changes nothing in exact
    arithmetic (paper §4)."""
    X = sample(n, m, seed=n * 100 + m)
    a = O.ns_standard(X)
    b = O.ns_gram(X, restart_after=restart)
    assert rel(b, a) <= 1e-10


def test_standard_ns_tall_input_is_transposed():
    X = sample(32, 8, seed=3)
    assert rel(O.ns_standard(X), O.ns_standard(X.T).T) <= 1e-13


@pytest.mark.parametrize("n,m", SHAPES)
def test_svd_identity(n, m):
    """X_T = U (p_T o..o p_1)(S) V^T for X0 = U S V^T (paper §2)."""
    X = sample(n, m, seed=7 * n + m)
    out = O.ns_gram(X)
    want, _ = O.polar_svd(X)
    assert rel(out, want) <= 1e-10
    # singular vectors are those of the polar factor: U^T O V is diagonal, > 0
    U, s, Vt = np.linalg.svd(X, full_matrices=False)
    D = U.T @ out @ Vt.T
    off = D - np.diag(np.diag(D))
    assert np.abs(off).max() <= 1e-10 * np.abs(np.diag(D)).max()
    assert np.all(np.diag(D) > 0)


def test_diagonal_input_closed_form():
    """A diagonal (padded) input maps each entry through the scalar polynomial
    composition; no SVD or matrix routine is involved in the expected value."""
    d = np.array([3.0, 1.0, 0.5, 0.25, 0.125, 2.0])
    n, m = d.size, 9
    X = np.zeros((n, m))
    X[np.arange(n), np.arange(n)] = d
    nrm = math.sqrt(sum(v * v for v in d)) + O.DEFAULT_EPS
    want = np.zeros((n, m))
    for i, v in enumerate(d):
        y = v / nrm
        for a, b, c in O.DEFAULT_COEFFS:
            y = a * y + b * y ** 3 + c * y ** 5
        want[i, i] = y
    for restart in [(), (2,)]:
        assert np.abs(O.ns_gram(X, restart_after=restart) - want).max() <= 1e-13
    assert np.abs(O.ns_standard(X) - want).max() <= 1e-13


def test_orthonormal_rows_scale_only():
    """Orthonormal rows times c: X0 = U/sqrt(n), output phi(1/sqrt(n)) U."""
    rng = np.random.default_rng(5)
    n, m = 8, 24
    Qm, _ = np.linalg.qr(rng.standard_normal((m, n)))
    U = Qm.T
    y = 1.0 / (math.sqrt(n) + O.DEFAULT_EPS / 3.7)  # c = 3.7 below
    for a, b, c in O.DEFAULT_COEFFS:
        y = a * y + b * y ** 3 + c * y ** 5
    assert rel(O.ns_gram(3.7 * U), y * U) <= 1e-12


def test_invariances():
    X = sample(12, 40, seed=11)
    base = O.ns_gram(X)
    P = np.random.default_rng(1).permutation(12)
    assert rel(O.ns_gram(X[P]), base[P]) <= 1e-12            # permutation equivariance
    assert rel(O.ns_gram(1e3 * X, eps=0.0), O.ns_gram(X, eps=0.0)) <= 1e-12   # scale
    assert rel(O.ns_standard(X.T), O.ns_standard(X).T) <= 1e-12                # transpose


def test_zero_input_gives_zero():
    Z = np.zeros((5, 9))
    assert np.all(O.ns_gram(Z) == 0)
    assert np.all(O.ns_standard(Z) == 0)


def test_phi_band_of_default_coefficients():
    """The default quintic maps [0.05, 1] into a band around 1 (it does not
    converge to 1; it only has to bring singular values near it)."""
    x = np.linspace(0.05, 1.0, 2000)
    y = O.compose_poly(x)
    assert y.min() > 0.6 and y.max() < 1.25


# ------------------------------------------------------------------- FLOPs
def _golden():
    rows = {}
    with open(os.path.join(GOLDEN, "flop_claims.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].split()
            if len(line) == 4:
                rows[line[0]] = float(line[3])
    return rows


def test_flop_tally_matches_pages():
    g = _golden()
    n, T, alpha = 16, 5, 4
    m = alpha * n
    X = sample(n, m, seed=2)
    tally = {}
    O.ns_gram(X, restart_after=(), flops=tally)
    gram_no_restart = sum(tally.values())
    assert gram_no_restart == (g["gram_coeff_T"] * T + g["gram_coeff_alpha"] * alpha
                               + g["gram_coeff_const"]) * n ** 3
    tally_r = {}
    O.ns_gram(X, restart_after=(2,), flops=tally_r)
    extra = sum(tally_r.values()) - gram_no_restart
    assert extra == (g["restart_extra_coeff_alpha"] * alpha + g["restart_extra_coeff_const"]) * n ** 3
    sym = O.ns_standard_flops(n, m, T, symmetric=True)
    dense = O.ns_standard_flops(n, m, T, symmetric=False)
    assert dense == (g["dense_standard_coeff_alpha"] * alpha + g["dense_standard_coeff_const"]) * n ** 3
    assert abs(100 * (1 - gram_no_restart / sym) - g["saving_vs_symmetric_standard_pct"]) <= 0.5
    assert abs(100 * (1 - gram_no_restart / dense) - g["saving_vs_dense_standard_pct"]) <= 0.5
    # rectangular multiplies: two in Gram NS without restart (the gram and the output)
    assert (tally["gram"] > 0) + (tally["rect"] > 0) == 1 + 1
    assert tally["gram"] == m * n * n and tally["rect"] == 2 * m * n * n
    assert g["gram_rect_gemms"] == 2 and g["standard_rect_gemms"] == 2 * T


# ------------------------------------------------------------------ selection
def rank_count_select(keys, k):
    """Brute force: row i is selected iff fewer than k rows beat it, where j
    beats i when key_j > key_i, or the keys tie and j < i (NaN counts as +inf)."""
    kk = [math.inf if math.isnan(v) else v for v in keys]
    sel = []
    for i, ki in enumerate(kk):
        beats = sum(1 for j, kj in enumerate(kk) if kj > ki or (kj == ki and j < i))
        if beats < k:
            sel.append(i)
    return sel


@pytest.mark.parametrize("seed", range(8))
def test_selection_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    keys = rng.integers(0, 6, size=n).astype(float)  # many ties
    if n > 3:
        keys[rng.integers(0, n)] = np.nan
    for k in range(1, n + 1):
        assert list(O.select_rows(keys, k)) == rank_count_select(list(keys), k)


def test_selection_ties_and_zero_rows():
    M = np.zeros((6, 4))
    M[1] = [1, -1, 2, 0]
    M[4] = [1, -1, 2, 0]      # duplicate of row 1
    M[3] = [0.5, 0, 0, 0]
    keys = O.l1_row_norms(M)
    assert list(O.select_rows(keys, 1)) == [1]
    assert list(O.select_rows(keys, 2)) == [1, 4]
    assert list(O.select_rows(keys, 3)) == [1, 3, 4]
    assert list(O.select_rows(keys, 4)) == [0, 1, 3, 4]   # zero rows: lowest index first


def test_l1_norms_exact():
    rng = np.random.default_rng(4)
    M = rng.standard_normal((5, 50)) * np.exp(8 * rng.standard_normal((5, 50)))
    got = O.l1_row_norms(M)
    for i in range(5):
        exact = sum(Fraction(abs(float(v))) for v in M[i])
        assert got[i] == float(exact)     # Fraction -> float is correctly rounded


def test_k_from_fraction():
    assert O.k_from_fraction(10, 0.25) == 3
    assert O.k_from_fraction(4096, 0.25) == 1024
    assert O.k_from_fraction(2048, 1 / 8) == 256
    assert O.k_from_fraction(5, 1.0) == 5
    assert O.k_from_fraction(1000, 1e-9) == 1
    assert O.k_from_fraction(10, 0.7) == 7 if Fraction(0.7) * 10 <= 7 else 8
    rng = np.random.default_rng(0)
    for _ in range(500):
        n = int(rng.integers(1, 20000))
        f = float(rng.random()) or 0.5
        k = O.k_from_fraction(n, f)
        exact = Fraction(f) * n
        assert 1 <= k <= n
        assert (k - 1 < exact <= k) or (k == 1 and exact <= 1)
    with pytest.raises(ValueError):
        O.k_from_fraction(10, 0.0)
    with pytest.raises(ValueError):
        O.k_from_fraction(10, 1.5)


# ------------------------------------------------------------------- rounding
def test_round_to_matches_library_casts():
    rng = np.random.default_rng(9)
    x = rng.standard_normal(200000) * np.exp(20 * rng.standard_normal(200000))
    x = np.concatenate([x, [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e-8, 6e-8, 3e38, 3.5e38, np.inf]])
    with np.errstate(over="ignore"):
        assert np.array_equal(O.round_to(x, "f32"), x.astype(np.float32).astype(np.float64))
        assert np.array_equal(O.round_to(x, "f16"), x.astype(np.float16).astype(np.float64))
    # bf16 from fp32 values (torch's cast is round-to-nearest-even from fp32)
    with np.errstate(over="ignore"):
        x32 = x.astype(np.float32)
    finite = np.isfinite(x32)
    tb = torch.from_numpy(x32[finite]).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_to(x32[finite].astype(np.float64), "bf16"), tb)


def _exact_round(v: Fraction, fmt: str) -> float:
    """Round a rational to fmt by enumeration of its two neighbours."""
    p, emin, _ = O.dion3.FORMATS[fmt]
    if v == 0:
        return 0.0
    s = 1 if v > 0 else -1
    a = abs(v)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    q = Fraction(2) ** (e - p + 1)
    lo = (a // q) * q
    hi = lo + q
    d_lo, d_hi = a - lo, hi - a
    if d_lo < d_hi:
        r = lo
    elif d_hi < d_lo:
        r = hi
    else:
        r = lo if (lo / q) % 2 == 0 else hi
    emax = O.dion3.FORMATS[fmt][2]
    if r > (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax:   # IEEE overflow
        return s * math.inf
    return s * float(r)


@pytest.mark.parametrize("fmt", ["f32", "bf16", "f16"])
def test_round_sum_exact(fmt):
    rng = np.random.default_rng(12)
    a = O.round_to(rng.standard_normal(3000) * np.exp(6 * rng.standard_normal(3000)), fmt)
    b = O.round_to(rng.standard_normal(3000) * np.exp(6 * rng.standard_normal(3000)), fmt)
    # crafted: exact midpoints plus a tiny tail so fp64 rounding hides the tail
    a2 = np.array([1.0, 1.0, -1.0, 2.0 ** 40])
    b2 = np.array([2.0 ** -24 + 2.0 ** -80, 2.0 ** -24 - 2.0 ** -80, -(2.0 ** -24 + 2.0 ** -80), 2.0 ** -30])
    a = np.concatenate([a, a2])
    b = np.concatenate([b, b2])
    big = 6e4 if fmt == "f16" else 1e30
    keep = np.isfinite(a) & np.isfinite(b) & (np.abs(a) < big) & (np.abs(b) < big)
    a, b = a[keep], b[keep]
    got = O.round_sum(a, b, fmt)
    for i in range(a.size):
        assert got[i] == _exact_round(Fraction(float(a[i])) + Fraction(float(b[i])), fmt), i


def test_momentum_decay_single_rounding_bf16():
    """m' = bf16(mu * m) rounded once: compare against exact rationals (an
    fp32 multiply followed by a cast would fail here)."""
    mu = O.f32(0.95)
    rng = np.random.default_rng(2)
    m = O.round_to(rng.standard_normal(20000), "bf16")
    got = O.round_to(mu * m, "bf16")
    want = np.array([_exact_round(Fraction(mu) * Fraction(float(v)), "bf16") for v in m])
    assert np.array_equal(got, want)
    twostep = O.round_to(O.round_to(mu * m, "f32"), "bf16")
    assert not np.array_equal(twostep, want)   # the double rounding really differs


# ------------------------------------------------------------------ full step
def test_f1_reduces_to_muon():
    """At f = 1 every row is selected and the step is Muon (paper §6; M0 = 0)."""
    rng = np.random.default_rng(21)
    n, m = 12, 30
    W = rng.standard_normal((n, m)) * 0.02
    Wm = W.copy()
    M = np.zeros((n, m))
    Mm = np.zeros((n, m))
    for _ in range(3):
        G = rng.standard_normal((n, m)) * np.exp(rng.standard_normal((n, 1)))
        out = O.dion3_step(W, M, G, k=n, mu=0.95, eta=0.02, wd=0.1, fmt="f64")
        W, M = out["W"], out["M"]
        Wm, Mm = O.muon_step(Wm, Mm, G, mu=0.95, eta=0.02, wd=0.1)
        assert rel(W, Wm) <= 1e-10
        assert rel(M, 0.95 * Mm) <= 1e-12  # stored M carries the mu of the last step


@pytest.mark.parametrize("fmt", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("shape", [(16, 40), (40, 16)])
def test_error_feedback_and_untouched_rows(fmt, shape):
    rng = np.random.default_rng(31)
    r, c = shape
    W = O.round_to(rng.standard_normal(shape) * 0.02, fmt)
    M = O.round_to(rng.standard_normal(shape), fmt)
    G = O.round_to(rng.standard_normal(shape) * np.exp(rng.standard_normal((r, 1))), fmt)
    k = 5
    out = O.dion3_step(W, M, G, k=k, mu=0.9, eta=0.05, fmt=fmt)
    axis = O.canonical_axis(r, c)
    Mc = O.momentum_accumulate(M, G, fmt)
    Wt, Mt, Mct = (W, out["M"], Mc) if axis == 0 else (W.T, out["M"].T, Mc.T)
    Wo = out["W"] if axis == 0 else out["W"].T
    sel = np.zeros(Wt.shape[0], bool)
    sel[out["idx"]] = True
    # unselected rows: W untouched, M = M + G (not decayed), both bit for bit
    assert np.array_equal(Wo[~sel], Wt[~sel])
    assert np.array_equal(Mt[~sel], Mct[~sel])
    # selected rows: M = mu M_hat (error feedback) and W moved by -eta O
    assert np.array_equal(Mt[sel], O.round_to(O.f32(0.9) * Mct[sel], fmt) if fmt != "f64" else 0.9 * Mct[sel])
    upd = (Wt[sel] - Wo[sel]) / 0.05
    tol = 1e-12 if fmt == "f64" else (1e-5 if fmt == "f32" else 0.05)
    assert rel(upd, out["O"]) <= tol
    assert len(out["idx"]) == k


def test_zero_selected_submatrix_leaves_w():
    W = np.full((4, 6), 0.5)
    M = np.zeros((4, 6))
    G = np.zeros((4, 6))
    out = O.dion3_step(W, M, G, k=2, mu=0.9, eta=0.1, fmt="bf16")
    assert np.all(out["O"] == 0)
    assert np.array_equal(out["W"], W)
    assert list(out["idx"]) == [0, 1]


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_apply_rows_fused_rounding_exact(wd):
    """Selected lines: w' = bf16(fp32(a - eta o)) with a = fp32(u w) (a = w when
    wd = 0), i.e. fp32 arithmetic and ONE cast back; unselected lines: bf16(a).
    Checked with exact rationals."""
    rng = np.random.default_rng(8)
    W = O.round_to(rng.standard_normal((6, 50)) * 0.02, "bf16")
    M = O.round_to(rng.standard_normal((6, 50)), "bf16")
    Ov = O.round_to(rng.standard_normal((3, 50)) * 0.05, "f16")
    idx = np.array([0, 2, 5])
    eta = O.f32(0.04)
    u = Fraction(_exact_round(1 - Fraction(eta) * Fraction(O.f32(wd)), "f32"))
    W2, _ = O.apply_rows(W, M, idx, Ov, 0.04, wd, 0.95, "bf16")
    sel = {int(i): r for r, i in enumerate(idx)}
    for i in range(6):
        for j in range(50):
            a = Fraction(float(W[i, j])) if wd == 0 else Fraction(_exact_round(u * Fraction(float(W[i, j])), "f32"))
            if i in sel:
                t = _exact_round(a - Fraction(eta) * Fraction(float(Ov[sel[i], j])), "f32")
            else:
                t = float(a)
            assert W2[i, j] == _exact_round(Fraction(t), "bf16"), (i, j)


def test_fp16_storage_model_within_tolerance():
    """Half-precision storage of every intermediate stays well inside the 3e-2
    tolerance on a Gaussian input with log-normal row scales."""
    X = sample(128, 512, seed=77)
    ref = O.ns_gram(X)
    assert rel(O.ns_gram_rounded(X, store="f16"), ref) < 1e-2
    assert rel(O.ns_gram_rounded(X, store="f32"), ref) < 1e-5


# The fp16 storage model, replayed in exact rational arithmetic: every product
# and every polynomial is formed exactly and each stored intermediate (the
# normalised input, R, Z, Q, Z R, Z R Z and the pass output) is rounded once to
# the storage format.  `skip` names one intermediate left unrounded and `fmt`
# may name the wrong format: the planted mistakes of the storage model.
STORED = ("x0", "R", "Z", "Q", "ZR", "ZRZ", "X")


def _rounded_gram_exact(X, coeffs, restart_after, fmt="f16", skip=None):
    n, m = X.shape
    rnd = lambda A, what: A if what == skip else [[Fraction(_exact_round(v, fmt)) for v in row] for row in A]
    mm = lambda A, B: [[sum((A[i][t] * B[t][j] for t in range(len(B))), Fraction(0)) for j in range(len(B[0]))]
                       for i in range(len(A))]
    tr = lambda A: [list(col) for col in zip(*A)]
    # the normalisation divides by the same fp64 norm the oracle computes
    nrm = Fraction(math.sqrt(float(np.sum(X * X))) + O.DEFAULT_EPS)
    Xf = rnd([[Fraction(float(v)) / nrm for v in row] for row in X], "x0")
    for t0, t1 in O.dion3._passes(len(coeffs), restart_after):
        R = rnd(mm(Xf, tr(Xf)), "R")
        Q = None
        for t in range(t0, t1):
            a, b, c = (Fraction(v) for v in coeffs[t])
            R2 = mm(R, R)
            Z = rnd([[(a if i == j else 0) + b * R[i][j] + c * R2[i][j] for j in range(n)] for i in range(n)], "Z")
            Q = Z if Q is None else rnd(mm(Q, Z), "Q")
            if t < t1 - 1:
                R = rnd(mm(rnd(mm(Z, R), "ZR"), Z), "ZRZ")
        Xf = rnd(mm(Q, Xf), "X")
    return np.array([[float(v) for v in row] for row in Xf])


def test_fp16_storage_model_is_exact_rounding():
    """ns_gram_rounded rounds every stored intermediate once, to fp16 (the
    pages switch the Gram iteration to float16, paper §4): on a 2 x 3 input with
    T = 3 and a restart after iteration 2 (so the Z R Z update, the Q Z
    product and the restart all occur), it equals the exact-rational replay bit
    for bit, and replays that skip any one rounding, or round to bf16 or not at
    all, differ from it."""
    X = np.array([[1.375, 0.5, 0.0], [-0.875, -0.75, -1.75]])
    coeffs, restart = O.DEFAULT_COEFFS[:3], (2,)
    want = _rounded_gram_exact(X, coeffs, restart)
    got = O.ns_gram_rounded(X, coeffs, restart, store="f16")
    assert np.array_equal(got, want)
    assert np.array_equal(O.round_to(got, "f16"), got)          # outputs are fp16 values
    # the planted mistakes of the storage model are each visible in the output
    for what in STORED:
        assert not np.array_equal(_rounded_gram_exact(X, coeffs, restart, skip=what), want), what
    assert not np.array_equal(_rounded_gram_exact(X, coeffs, restart, fmt="bf16"), want)
    assert not np.array_equal(O.ns_gram_rounded(X, coeffs, restart, store="bf16"), want)
    assert not np.array_equal(O.ns_gram_rounded(X, coeffs, restart, store="f64"), want)
    # and with fp32 storage the oracle matches the fp32 replay
    assert np.array_equal(O.ns_gram_rounded(X, coeffs, restart, store="f32"),
                          _rounded_gram_exact(X, coeffs, restart, fmt="f32"))


# ------------------------------------------------------ planted mistakes fail
def _gram_variant(X, mistake, coeffs=O.DEFAULT_COEFFS, restart_after=(2,)):
    X = O.frobenius_normalize(X)
    n = X.shape[0]
    I = np.eye(n)
    for t0, t1 in O.dion3._passes(len(coeffs), restart_after):
        R = X @ X.T
        Q = None
        for t in range(t0, t1):
            a, b, c = coeffs[t]
            if mistake == "drop_c":
                Z = a * I + b * R
            elif mistake == "sign_b":
                Z = a * I - b * R + c * (R @ R)
            else:
                Z = a * I + b * R + c * (R @ R)
            Q = Z if Q is None else Q @ Z
            if t < t1 - 1:
                R = Z @ R if mistake == "one_sided_R" else Z @ R @ Z
        X = (X.T @ Q).T if mistake == "transpose_X" and n == X.shape[1] else Q @ X
        if mistake == "no_restart_rebuild":
            break
    return X


@pytest.mark.parametrize("mistake", ["drop_c", "sign_b", "one_sided_R", "no_restart_rebuild"])
def test_planted_mistakes_are_caught(mistake):
    X = sample(8, 32, seed=4)
    good = O.ns_standard(X)
    bad = _gram_variant(X, mistake)
    ok_gram = rel(bad, good) <= 1e-10
    svd, _ = O.polar_svd(X)
    ok_svd = rel(bad, svd) <= 1e-10
    assert not (ok_gram and ok_svd)
    # and the correct variant passes both
    fine = _gram_variant(X, "none")
    assert rel(fine, good) <= 1e-10 and rel(fine, svd) <= 1e-10


# ------------------------------------------------------------ NorMuon flavour
@pytest.mark.parametrize("shape", [(6, 20), (16, 64)])
def test_normuon_equal_moments_leave_o_unchanged(shape):
    """beta2 = 1 keeps v; equal v on every row scales all rows alike, and the
    Frobenius rescale undoes the common factor: O_hat = O."""
    Ob = sample(*shape, seed=11)
    v = np.full(shape[0], 0.37)
    Oh, vn = O.normuon_scale(Ob, v, beta2=1.0, eps=1e-3)
    assert np.array_equal(vn, v)
    assert rel(Oh, Ob) <= 1e-14


@pytest.mark.parametrize("beta2", [0.0, 0.5, 0.95])
def test_normuon_balances_row_norms(beta2):
    """v = 0 and eps = 0: the new moment is (1 - beta2) times each row's mean
    square, so every row of O_hat has the same norm, and ||O_hat||_F = ||O||_F."""
    Ob = sample(8, 32, seed=12)          # rows of very different norms
    Oh, vn = O.normuon_scale(Ob, np.zeros(8), beta2=beta2, eps=0.0)
    rows = np.linalg.norm(Oh, axis=1)
    assert np.ptp(rows) <= 1e-12 * rows.max()
    assert abs(np.linalg.norm(Oh) - np.linalg.norm(Ob)) <= 1e-12 * np.linalg.norm(Ob)
    assert rel(vn, (1.0 - beta2) * np.mean(Ob * Ob, axis=1)) <= 1e-15


def test_normuon_moment_is_an_ema():
    """beta2 = 0 makes v this step's row mean square; beta2 = 1 keeps it."""
    Ob = sample(5, 9, seed=13)
    v = np.arange(1.0, 6.0)
    assert rel(O.normuon_scale(Ob, v, beta2=0.0)[1], np.mean(Ob ** 2, axis=1)) <= 1e-15
    assert np.array_equal(O.normuon_scale(Ob, v, beta2=1.0)[1], v)


@pytest.mark.parametrize("mistake", ["no_rescale", "no_row_scale", "sum_not_mean"])
def test_normuon_planted_mistakes_are_caught(mistake):
    def variant(Ob, v, beta2, eps):
        q = np.sum(Ob * Ob, axis=1) / (1.0 if mistake == "sum_not_mean" else Ob.shape[1])
        vn = beta2 * v + (1.0 - beta2) * q
        d = np.ones_like(vn) if mistake == "no_row_scale" else 1.0 / (np.sqrt(vn) + eps)
        Oh = Ob * d[:, None]
        if mistake != "no_rescale":
            Oh *= np.linalg.norm(Ob) / np.linalg.norm(Oh)
        return Oh, vn
    Ob = 3.0 * sample(8, 32, seed=14)
    ok = []
    # the three pins above, applied to the variant
    Oh, vn = variant(Ob, np.full(8, 0.37), 1.0, 1e-3)
    ok.append(rel(Oh, Ob) <= 1e-14)
    Oh, vn = variant(Ob, np.zeros(8), 0.5, 0.0)
    rows = np.linalg.norm(Oh, axis=1)
    ok.append(np.ptp(rows) <= 1e-12 * rows.max()
              and abs(np.linalg.norm(Oh) - np.linalg.norm(Ob)) <= 1e-12 * np.linalg.norm(Ob))
    ok.append(rel(variant(Ob, np.arange(1.0, 9.0), 0.0, 1e-8)[1], np.mean(Ob ** 2, axis=1)) <= 1e-15)
    assert not all(ok)


def test_normuon_step_untouched_lines_and_moments():
    """The NorMuon step changes V only on the selected lines, and W and M only
    on the selected lines (canonical orientation)."""
    rng = np.random.default_rng(15)
    W, M, G = rng.standard_normal((3, 24, 10))        # rows > cols: columns selected
    V = np.abs(rng.standard_normal(10))
    out = O.dion3_step(W, M, G, k=4, mu=0.9, eta=0.1, V=V)
    sel = np.zeros(10, dtype=bool)
    sel[out["idx"]] = True
    assert np.array_equal(out["V"][~sel], V[~sel])
    assert np.all(out["V"][sel] != V[sel])
    assert np.array_equal(out["W"][:, ~sel], W[:, ~sel])
    assert np.array_equal(out["M"][:, ~sel], (M + G)[:, ~sel])
    assert abs(np.linalg.norm(out["O_hat"]) - np.linalg.norm(out["O"])) <= 1e-12 * np.linalg.norm(out["O"])


def test_restart_keeps_fp16_gram_ns_accurate():
    """Why the iteration restarts ("Dion3: Full-Stack Orthogonal Updates",
    Section 4 and Appendix B: half-precision storage makes the Gram iteration
    drift, restarting from a fresh Gram matrix repairs it).  On inputs whose
    singular values span 3 to 6 decades, the fp16 storage model without a
    restart ends far from the fp64 iteration (relative error > 0.2), with the
    restart after iteration 2 about ten times closer (< 4e-2), and in fp64
    storage both are the same map (the divergence is rounding, not algebra)."""
    for smin, seed in [(1e-3, 1), (1e-6, 2)]:
        r = np.random.default_rng(seed)
        n, m = 32, 128
        U, _ = np.linalg.qr(r.standard_normal((n, n)))
        V, _ = np.linalg.qr(r.standard_normal((m, n)))
        X = (U * np.logspace(0, np.log10(smin), n)) @ V.T
        ref = O.ns_standard(X)
        err = lambda Y: np.linalg.norm(Y - ref) / np.linalg.norm(ref)
        e_plain = err(O.ns_gram_rounded(X, restart_after=(), store="f16"))
        e_restart = err(O.ns_gram_rounded(X, restart_after=(2,), store="f16"))
        assert e_plain > 0.2 and e_restart < 4e-2 and e_plain > 8 * e_restart, (smin, e_plain, e_restart)
        assert err(O.ns_gram_rounded(X, restart_after=(), store="f64")) < 1e-10
        assert err(O.ns_gram_rounded(X, restart_after=(2,), store="f64")) < 1e-10
