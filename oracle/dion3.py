"""Plain, slow, fp64 CPU oracle for the Dion3 update of one matrix parameter.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code with the HIP library and imports
nothing from the product package.

Sources (all citations are to the pages describing the method; the section
numbers of the paper text are inferred from its own cross-references because
its headings were lost):
  * "Dion3: Full-Stack Orthogonal Updates", paper text  -> cited as [paper §n]
  * "Dion3: Full-Stack Orthogonal Updates", agihunt summary -> [summary]

What is computed, in the pages' order and notation:
  1. momentum accumulation  M <- M + G                     [paper §6, footnote 4
                                                             of the f=1 paragraph]
  2. l1 norm of every row of M, keep the k = ceil(f n) rows with the largest
     norm                                                  [paper §6, selection]
  3. O = Newton-Schulz approximation of polar(M[S, :]), run as Gram
     Newton-Schulz with a restart after iteration 2        [paper §4]
  4. W[S, :] <- W[S, :] - eta O (weight decay, if on, on all rows first), with
     the fp32 arithmetic and a single cast back           [paper §6, fused
                                                             weight update]
  5. error feedback: M <- mu M_hat + (M - M_hat), i.e. only the selected rows
     of M are multiplied by mu                              [paper §6]

Readings of points the pages leave open (each is listed in the design notes):
  * Orientation: the selection axis is the smaller dimension (rows on a tie);
    a matrix with more rows than columns is handled through its transpose
    [paper §6, choice of rows vs columns].
  * The Newton-Schulz coefficient table is a parameter; DEFAULT_COEFFS is the
    fixed quintic of Muon's public write-up (the pages name the source but do
    not print values).  parity unpinned for the coefficient VALUES only.
  * X0 = X / (||X||_F + eps) with eps = 1e-7 [paper §2 normalisation; the guard
    is ours].
  * Every rounding is round-to-nearest-even of the exact real result.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

# --------------------------------------------------------------------------
# Coefficients.  p_t(x) = a_t x + b_t x^3 + c_t x^5   [paper §2, SVD view of NS]
# Default: Muon's published fixed quintic, the same for all T iterations.
# --------------------------------------------------------------------------
MUON_QUINTIC = (3.4445, -4.7750, 2.0315)
DEFAULT_T = 5
DEFAULT_COEFFS = tuple(MUON_QUINTIC for _ in range(DEFAULT_T))
DEFAULT_RESTART_AFTER = (2,)        # "restart at iteration 3" [paper §4]
DEFAULT_EPS = 1e-7

# --------------------------------------------------------------------------
# Rounding: IEEE round-to-nearest-even of an exact real value to a binary
# format with p significand bits and minimum normal exponent emin.
# --------------------------------------------------------------------------
FORMATS = {
    # name: (precision p, emin, emax)
    "f64": (53, -1022, 1023),
    "f32": (24, -126, 127),
    "bf16": (8, -126, 127),
    "f16": (11, -14, 15),
}


def _quantum(x: np.ndarray, fmt: str) -> np.ndarray:
    """Spacing of `fmt` values in the binade of x (subnormal spacing below)."""
    p, emin, _ = FORMATS[fmt]
    _, e = np.frexp(x)                 # x = f 2^e with 0.5 <= |f| < 1
    lead = np.maximum(e.astype(np.int64) - 1, emin)
    return np.ldexp(np.ones_like(x, dtype=np.float64), (lead - (p - 1)).astype(np.int32))


def round_to(x, fmt: str) -> np.ndarray:
    """Round fp64 values, taken as exact reals, to the nearest `fmt` value.

    Ties go to the even neighbour; values past the largest finite number
    (by at least half a unit) become infinities; NaN stays NaN.  The result is
    returned as float64 holding an exactly representable `fmt` value."""
    x = np.asarray(x, dtype=np.float64)
    if fmt == "f64":
        return x.copy()
    p, _, emax = FORMATS[fmt]
    with np.errstate(invalid="ignore", over="ignore"):
        q = _quantum(x, fmt)
        y = np.rint(x / q) * q                      # np.rint rounds half to even
        big = (2.0 - 2.0 ** (1 - p)) * 2.0 ** emax  # largest finite value
        y = np.where(np.abs(y) > big, np.copysign(np.inf, x), y)
    return y


def round_sum(a, b, fmt: str) -> np.ndarray:
    """Round the exact real a + b (a, b fp64 values) once to `fmt`.

    a + b is split error-free into s + err (Knuth's two-sum).  Rounding s is
    already the correct rounding of s + err unless s lies exactly half-way
    between two `fmt` neighbours; there the sign of err picks the side."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        s = a + b
        bb = s - a
        err = (a - (s - bb)) + (b - bb)
        r = round_to(s, fmt)
        if fmt == "f64":
            return r
        q = _quantum(s, fmt)
        t = s / q
        mid = np.isfinite(s) & (t - np.floor(t) == 0.5) & (err != 0)
        if np.any(mid):
            up = np.ceil(t) * q
            dn = np.floor(t) * q
            r = np.where(mid, np.where(err > 0, up, dn), r)
    return r


# --------------------------------------------------------------------------
# Step 1: momentum accumulation, M <- M + G  [paper §6, f=1 paragraph and its
# footnote: Newton-Schulz sees M + G, damping comes after the update]
# --------------------------------------------------------------------------
def momentum_accumulate(M, G, fmt: str) -> np.ndarray:
    return round_sum(M, G, fmt)


# --------------------------------------------------------------------------
# Step 2: l1 row norms and top-k selection  [paper §6, selection strategy;
# summary: k = ceil(f n) rows of largest l1 norm]
# --------------------------------------------------------------------------
def k_from_fraction(n: int, f: float) -> int:
    """k = ceil(f n) of the exact product of the given float f and n, in [1, n]."""
    if not (n >= 1) or not (0.0 < f <= 1.0):
        raise ValueError("need n >= 1 and 0 < f <= 1")
    k = math.ceil(Fraction(f) * n)
    return max(1, min(n, k))


def l1_row_norms(M) -> np.ndarray:
    """key_i = sum_j |M_ij|, each an exactly rounded fp64 sum (math.fsum)."""
    M = np.asarray(M, dtype=np.float64)
    return np.array([math.fsum(np.abs(row)) for row in M], dtype=np.float64)


def select_rows(keys, k: int) -> np.ndarray:
    """Indices of the k largest keys, ties to the lower index, listed ascending.

    A NaN key orders as +infinity, so a non-finite row is always selected."""
    keys = np.asarray(keys, dtype=np.float64)
    n = keys.shape[0]
    if not 1 <= k <= n:
        raise ValueError("k out of range")
    kk = np.where(np.isnan(keys), np.inf, keys)
    order = np.lexsort((np.arange(n), -kk))   # primary: key descending; then index
    return np.sort(order[:k]).astype(np.int64)


# --------------------------------------------------------------------------
# Step 3: Newton-Schulz  [paper §2 (Algorithm 1 and its SVD view), §4 (Gram
# Newton-Schulz, restart)]
# --------------------------------------------------------------------------
def frobenius_normalize(X, eps: float = DEFAULT_EPS) -> np.ndarray:
    X = np.asarray(X, dtype=np.float64)
    return X / (math.sqrt(float(np.sum(X * X))) + eps)


def ns_standard(X, coeffs=DEFAULT_COEFFS, eps: float = DEFAULT_EPS) -> np.ndarray:
    """Standard Newton-Schulz (paper §2): on X0 = X/||X||_F (n <= m, transpose
    otherwise) each iteration forms A = X X^T, B = b A + c A^2, X <- a X + B X."""
    X = np.asarray(X, dtype=np.float64)
    flip = X.shape[0] > X.shape[1]
    if flip:
        X = X.T
    X = frobenius_normalize(X, eps)
    for a, b, c in coeffs:
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if flip else X


def _passes(T: int, restart_after) -> list[tuple[int, int]]:
    cuts = sorted({int(r) for r in restart_after if 0 < int(r) < T})
    bounds = [0] + cuts + [T]
    return [(bounds[i], bounds[i + 1]) for i in range(len(bounds) - 1)]


def ns_gram(X, coeffs=DEFAULT_COEFFS, restart_after=DEFAULT_RESTART_AFTER,
            eps: float = DEFAULT_EPS, flops: dict | None = None) -> np.ndarray:
    """Gram Newton-Schulz with restarts (paper §4), for n <= m.

    Within one pass, on R = X X^T:
        Z_t = a_t I + b_t R + c_t R^2
        Q_t = Q_{t-1} Z_t            (Q = Z_t on the pass's first iteration)
        R_t = Z_t R_{t-1} Z_t        (skipped on the pass's last iteration)
    and the pass ends with X <- Q X.  A restart starts a new pass on the
    current X (the Gram matrix is rebuilt and Q reset to the identity).
    Since X_t = Z_t X_{t-1}, this is standard Newton-Schulz rewritten.

    If `flops` is a dict, products are tallied with the pages' convention:
    a symmetric k x k product costs k^3, X X^T costs m k^2 and Q X 2 m k^2."""
    X = np.asarray(X, dtype=np.float64)
    n, m = X.shape
    if n > m:
        raise ValueError("Gram Newton-Schulz expects n <= m (transpose first)")
    X = frobenius_normalize(X, eps)
    I = np.eye(n)
    tally = flops if flops is not None else {}
    tally.setdefault("gram", 0)
    tally.setdefault("square", 0)
    tally.setdefault("rect", 0)
    for t0, t1 in _passes(len(coeffs), restart_after):
        R = X @ X.T
        tally["gram"] += m * n * n
        Q = None
        for t in range(t0, t1):
            a, b, c = coeffs[t]
            Z = a * I + b * R + c * (R @ R)
            tally["square"] += n ** 3
            if Q is None:
                Q = Z
            else:
                Q = Q @ Z
                tally["square"] += n ** 3
            if t < t1 - 1:
                R = Z @ R @ Z
                tally["square"] += 2 * n ** 3
        X = Q @ X
        tally["rect"] += 2 * m * n * n
    return X


def ns_standard_flops(n: int, m: int, T: int, symmetric: bool) -> int:
    """Cost of standard NS as the pages count it (paper §2 and §3): per
    iteration X X^T, A^2 and B X; symmetric products cost half."""
    if symmetric:
        return T * (m * n * n + n ** 3 + 2 * m * n * n)
    return T * (2 * m * n * n + 2 * n ** 3 + 2 * m * n * n)


def compose_poly(x, coeffs=DEFAULT_COEFFS) -> np.ndarray:
    """(p_T o ... o p_1)(x) on scalars, p_t(x) = a_t x + b_t x^3 + c_t x^5."""
    y = np.asarray(x, dtype=np.float64)
    for a, b, c in coeffs:
        y = a * y + b * y ** 3 + c * y ** 5
    return y


def polar_svd(X, coeffs=DEFAULT_COEFFS, eps: float = DEFAULT_EPS):
    """SVD view of Newton-Schulz (paper §2): with X0 = U S V^T, the T-step
    output is U (p_T o..o p_1)(S) V^T, and polar(X) = U V^T.
    Returns (U phi(S) V^T, U V^T)."""
    X0 = frobenius_normalize(X, eps)
    U, s, Vt = np.linalg.svd(X0, full_matrices=False)
    return (U * compose_poly(s, coeffs)) @ Vt, U @ Vt


# --------------------------------------------------------------------------
# Step 3 under a half-precision storage model: every stored intermediate is
# rounded to `store` between exact products (a model of fp16 operands with
# wide accumulation).  Used to predict the error floor of the fp16 path.
# --------------------------------------------------------------------------
def ns_gram_rounded(X, coeffs=DEFAULT_COEFFS, restart_after=DEFAULT_RESTART_AFTER,
                    eps: float = DEFAULT_EPS, store: str = "f16") -> np.ndarray:
    X = np.asarray(X, dtype=np.float64)
    n, _ = X.shape
    rnd = lambda A: round_to(A, store)
    X = rnd(frobenius_normalize(X, eps))
    I = np.eye(n)
    for t0, t1 in _passes(len(coeffs), restart_after):
        R = rnd(X @ X.T)
        Q = None
        for t in range(t0, t1):
            a, b, c = coeffs[t]
            Z = rnd(a * I + b * R + c * (R @ R))
            Q = Z if Q is None else rnd(Q @ Z)
            if t < t1 - 1:
                R = rnd(rnd(Z @ R) @ Z)
        X = rnd(Q @ X)
    return X


# --------------------------------------------------------------------------
# Steps 4 and 5: weight update with a single rounding, error feedback
# [paper §6: weight decay on all rows first; the fused update is evaluated in
# fp32 and cast back once; only selected momentum rows are decayed by mu]
# --------------------------------------------------------------------------
def f32(v: float) -> float:
    """The fp32 value nearest to v (scalars enter the update as fp32)."""
    return float(round_to(np.float64(v), "f32"))


def apply_rows(W, M, idx, O, eta: float, wd: float, mu: float, fmt: str):
    """Return (W', M') for rows idx of W and M (canonical orientation).

    Arithmetic is fp32 with one rounding per operation as the pages describe:
      u  = fp32(1 - eta*wd)                       (a scalar)
      a  = fp32(u * w)                            (all rows, only if wd != 0)
      w' = fmt(fp32(a - eta*o))                   (selected rows)
      m' = fmt(mu * m)                            (selected rows, one rounding)
    eta, mu are fp32 values; eta*o and u*w are exact in fp64."""
    W = np.array(W, dtype=np.float64)
    M = np.array(M, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    if fmt == "f64":
        # exact-arithmetic model (no storage rounding), used by the algebraic pins
        W = (1.0 - eta * wd) * W
        W[idx] = W[idx] - eta * np.asarray(O, dtype=np.float64)
        M[idx] = mu * M[idx]
        return W, M
    eta32, mu32 = f32(eta), f32(mu)
    A = W
    if wd != 0.0:
        u = f32(1.0 - eta32 * f32(wd))
        A = round_to(u * W, "f32")          # fp32 value of the decayed weights
    upd = round_sum(A[idx], -eta32 * np.asarray(O, dtype=np.float64), "f32")
    W = round_to(A, fmt)                    # unselected lines: one cast of u*w
    W[idx] = round_to(upd, fmt)             # selected lines: one cast of u*w - eta*o
    M[idx] = round_to(mu32 * M[idx], fmt)
    return W, M


# --------------------------------------------------------------------------
# NorMuon flavour  [paper §2 (NorMuon divides each row of the orthogonalised
# update by the root of that row's second moment, then rescales the update so
# that its Frobenius norm is Muon's), §6 (the flavour updates the second
# moments of the selected rows and rescales O; the normalisation runs in
# fp32)].  The pages' equation and listing are missing from the extracted
# text; this is the plainest reading of the prose:
#   q_i = mean_j O_ij^2;   v_i <- beta2 v_i + (1 - beta2) q_i;
#   O_hat_i = O_i / (sqrt(v_i) + eps);   O_hat <- O_hat ||O||_F / ||O_hat||_F
# beta2 and eps are parameters (no values survive in the text); no bias
# correction.
# --------------------------------------------------------------------------
DEFAULT_BETA2 = 0.95
DEFAULT_NORMUON_EPS = 1e-8


def normuon_scale(O, v, beta2: float = DEFAULT_BETA2, eps: float = DEFAULT_NORMUON_EPS):
    """(O_hat, v_new) for the k selected rows O (k x m) and their second
    moments v (k); exact arithmetic in fp64."""
    O = np.asarray(O, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q = np.sum(O * O, axis=1) / O.shape[1]
    v_new = beta2 * v + (1.0 - beta2) * q
    d = 1.0 / (np.sqrt(v_new) + eps)
    Oh = O * d[:, None]
    nh = math.sqrt(float(np.sum(Oh * Oh)))
    r = math.sqrt(float(np.sum(O * O))) / nh if nh > 0.0 else 1.0
    return Oh * r, v_new


# --------------------------------------------------------------------------
# The whole step on one matrix
# --------------------------------------------------------------------------
def canonical_axis(rows: int, cols: int, sel_axis: int = -1) -> int:
    """0: select rows; 1: select columns (the smaller dimension, rows on a tie)."""
    if sel_axis in (0, 1):
        return sel_axis
    return 0 if rows <= cols else 1


def dion3_step(W, M, G, *, k: int, mu: float, eta: float, wd: float = 0.0,
               coeffs=DEFAULT_COEFFS, restart_after=DEFAULT_RESTART_AFTER,
               eps: float = DEFAULT_EPS, fmt: str = "f64", sel_axis: int = -1,
               ns=None, keys_exact: bool = True, V=None,
               beta2: float = DEFAULT_BETA2, nm_eps: float = DEFAULT_NORMUON_EPS):
    """One Dion3 step on a single matrix: the Muon flavour, or the NorMuon
    flavour when V (the second moment of every line of the selection axis) is
    given.

    Returns dict(W, M, idx, O, keys[, V, O_hat]) with W, M in stored
    orientation and idx, O, keys, V, O_hat in canonical orientation (selected
    axis first)."""
    W = np.asarray(W, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    axis = canonical_axis(W.shape[0], W.shape[1], sel_axis)
    if axis == 1:
        W, M, G = W.T, M.T, G.T
    M = momentum_accumulate(M, G, fmt)
    keys = l1_row_norms(M) if keys_exact else np.sum(np.abs(M), axis=1)
    idx = select_rows(keys, k)
    X = M[idx]
    if ns is None:
        # aspect ratio 1 (square selected submatrix): standard Newton-Schulz,
        # the pages' fall-back (paper §4); Gram Newton-Schulz otherwise
        O = ns_standard(X, coeffs, eps) if X.shape[0] == X.shape[1] else ns_gram(X, coeffs, restart_after, eps)
    else:
        O = ns(X)
    out = {"idx": idx, "O": O, "keys": keys}
    U = O
    if V is not None:
        V = np.array(V, dtype=np.float64)
        U, V[idx] = normuon_scale(O, V[idx], beta2, nm_eps)
        out["V"], out["O_hat"] = V, U
    W, M = apply_rows(W, M, idx, U, eta, wd, mu, fmt)
    if axis == 1:
        W, M = W.T, M.T
    out["W"], out["M"] = W, M
    return out


def muon_step(W, M, G, *, mu: float, eta: float, wd: float = 0.0,
              coeffs=DEFAULT_COEFFS, eps: float = DEFAULT_EPS):
    """Plain Muon in exact arithmetic (paper §2): M <- mu M + G,
    W <- (1 - eta wd) W - eta NS(M), with standard Newton-Schulz."""
    M = mu * np.asarray(M, dtype=np.float64) + np.asarray(G, dtype=np.float64)
    W = (1.0 - eta * wd) * np.asarray(W, dtype=np.float64) - eta * ns_standard(M, coeffs, eps)
    return W, M
