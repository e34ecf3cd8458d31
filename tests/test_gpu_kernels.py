"""GPU parity of each C entry point against the CPU oracle (through the C ABI).

Sizes span several tiles and ragged tails; indices, M and the update rounding
are compared bit for bit, floating-point products within tolerances derived
from the arithmetic (fp32 accumulation, one rounding to the output type)."""

import numpy as np
import pytest
import torch

import oracle as O
from helpers import bits, np_bits, rel_fro, to64
from muon_momentum_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def d():
    import muon_momentum_amd.dion3 as mod
    return mod


TD = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
# normwise tolerance for products stored in the output type (one rounding of
# the result plus fp32 accumulation): well below the unit roundoff x 4
TOL = {"f16": 2e-3, "bf16": 1.2e-2, "f32": 2e-5}


# ------------------------------------------------------- symmetric products
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("b,n,kd", [(1, 256, 512), (3, 128, 1024), (2, 200, 300), (1, 384, 136), (1, 33, 7)])
def test_syrk(d, dt, b, n, kd):
    A = synth.dense(n, kd, b, dtype=dt, device=DEV, seed=n + kd)
    C = torch.full((b, n, n), float("nan"), dtype=TD[dt], device=DEV)
    d.dion3_syrk(A, C, alpha=1.0, beta=0.0)
    torch.cuda.synchronize()
    a = to64(A)
    ref = a @ a.transpose(0, 2, 1)
    got = to64(C)
    assert np.all(np.isfinite(got))
    cb = bits(C)
    assert np.array_equal(cb, cb.transpose(0, 2, 1))       # exactly symmetric
    assert rel_fro(got, ref) <= TOL[dt]


@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_syrk_beta(d, dt):
    b, n, kd = 2, 256, 256
    A = synth.dense(n, kd, b, dtype=dt, device=DEV, seed=3)
    C0 = synth.symmetric(n, b, dtype=dt, device=DEV, seed=4)
    C = C0.clone()
    d.dion3_syrk(A, C, alpha=0.5, beta=-2.0)
    torch.cuda.synchronize()
    a = to64(A)
    ref = 0.5 * a @ a.transpose(0, 2, 1) - 2.0 * to64(C0)
    assert rel_fro(to64(C), ref) <= TOL[dt]
    cb = bits(C)
    assert np.array_equal(cb, cb.transpose(0, 2, 1))


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("b,n", [(1, 256), (2, 384), (3, 200), (1, 130)])
def test_sym_sq_add(d, dt, b, n):
    A = synth.symmetric(n, b, dtype=dt, device=DEV, seed=10 + n)
    B = synth.symmetric(n, b, dtype=dt, device=DEV, seed=20 + n)
    C = torch.empty_like(A)
    al, be, ga = 2.0315, -4.7750, 3.4445
    d.dion3_sym_sq_add(A, B, C, alpha=al, beta=be, gamma=ga)
    torch.cuda.synchronize()
    a, bb = to64(A), to64(B)
    ref = al * a @ a + be * bb + ga * np.eye(n)[None]
    assert rel_fro(to64(C), ref) <= TOL[dt]
    cb = bits(C)
    assert np.array_equal(cb, cb.transpose(0, 2, 1))


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("b,n", [(1, 256), (2, 200)])
def test_sym_mul_commuting(d, dt, b, n):
    """A and B are polynomials in one symmetric matrix, so A B is symmetric."""
    S = to64(synth.symmetric(n, b, dtype="f32", device="cpu", seed=5))
    A64 = 1.5 * np.eye(n)[None] + 0.7 * S
    B64 = 0.3 * np.eye(n)[None] - 0.2 * S + 0.4 * S @ S
    A = torch.from_numpy(A64).to(TD[dt]).to(DEV)
    B = torch.from_numpy(B64).to(TD[dt]).to(DEV)
    C = torch.empty_like(A)
    d.dion3_sym_mul(A, B, C, alpha=1.0)
    torch.cuda.synchronize()
    a, bb = to64(A), to64(B)
    ref = a @ bb
    ref = np.tril(ref) + np.tril(ref, -1).transpose(0, 2, 1)   # the lower triangle, mirrored
    assert rel_fro(to64(C), ref) <= TOL[dt]
    cb = bits(C)
    assert np.array_equal(cb, cb.transpose(0, 2, 1))


@pytest.mark.parametrize("dt,odt", [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("b,k,m", [(1, 256, 1024), (2, 128, 640), (2, 100, 300), (1, 64, 2048)])
def test_gemm_qx(d, dt, odt, b, k, m):
    Q = synth.symmetric(k, b, dtype=dt, device=DEV, seed=k)
    X = synth.dense(k, m, b, dtype=dt, device=DEV, seed=m)
    Y = torch.empty(b, k, m, dtype=TD[odt], device=DEV)
    d.dion3_gemm(Q, X, Y, alpha=1.0)
    torch.cuda.synchronize()
    ref = to64(Q) @ to64(X)
    assert rel_fro(to64(Y), ref) <= TOL[odt if odt != "f32" else dt]


# --------------------------------------------------- momentum and selection
def _rowsel_case(d, rows, cols, batch, dt, k, sel_axis=-1, G=None, M0=None):
    if G is None:
        G = synth.gradient(rows, cols, batch, dtype=dt, device=DEV, group_seed=rows + cols, sel_axis=sel_axis)
    M = (M0.clone() if M0 is not None
         else synth.gradient(rows, cols, batch, dtype=dt, device=DEV, group_seed=7, step=3, sel_axis=sel_axis))
    Mh, Gh = to64(M), to64(G)
    n, m, axis = d.dion3_canonical(d.make_group(M, sel_axis))
    idx = torch.full((batch, k), -1, dtype=torch.int32, device=DEV)
    keys = torch.empty(batch, n, dtype=torch.float64, device=DEV)
    sqn = torch.empty(batch, dtype=torch.float64, device=DEV)
    d.dion3_momentum_rowsel(M, G, k, idx, keys, sqn, sel_axis=sel_axis)
    torch.cuda.synchronize()
    return M, Mh, Gh, idx.cpu().numpy(), keys.cpu().numpy(), sqn.cpu().numpy(), axis


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols,batch,f,axis", [
    (256, 1024, 1, 1.0, -1), (300, 1000, 2, 0.25, -1), (200, 1001, 2, 0.125, -1),
    (600, 200, 2, 0.25, -1), (1100, 520, 1, 0.5, -1), (2500, 2600, 1, 0.25, -1),
    (257, 300, 3, 0.25, 1), (64, 64, 4, 0.5, -1)])
def test_momentum_rowsel(d, dt, rows, cols, batch, f, axis):
    n = (rows if rows <= cols else cols) if axis == -1 else (rows if axis == 0 else cols)
    k = O.k_from_fraction(n, f)
    M, Mh, Gh, idx, keys, sqn, ax = _rowsel_case(d, rows, cols, batch, dt, k, sel_axis=axis)
    for b in range(batch):
        Mref = O.momentum_accumulate(Mh[b], Gh[b], dt)
        assert np.array_equal(bits(M[b]), np_bits(Mref, TD[dt]))          # M bit-exact
        Mc = Mref if ax == 0 else Mref.T
        kref = O.l1_row_norms(Mc)
        assert np.max(np.abs(keys[b] - kref) / np.maximum(kref, 1e-300)) <= 1e-12
        sref = O.select_rows(kref, k)
        # boundary gap: the k-th and (k+1)-th keys must be clearly separated
        srt = np.sort(kref)[::-1]
        if k < n:
            assert (srt[k - 1] - srt[k]) / srt[k - 1] > 1e-12
        assert np.array_equal(idx[b], sref)                                 # indices bit-exact
        sq = float(np.sum(Mc[sref] ** 2))
        assert abs(sqn[b] - sq) <= 1e-12 * sq


def test_bf16_rounding_special_values(d):
    """The bf16 rounding of the library's kernels on the momentum pass: exact
    ties (to even), neighbours of ties, overflow to infinity, subnormal sums
    and signed zeros equal the oracle's round-once sum bit for bit; a NaN
    input leaves that NaN quieted, sign and upper payload bits kept (bf16 bits
    0x7fa1 -> 0x7fe1)."""
    pairs = [  # (M bits, G bits) in bf16
        (0x3F80, 0x3B80), (0x3F81, 0x3B80), (0xBF81, 0xBB80), (0x3F80, 0x3B81),
        (0x3F81, 0x3B7F), (0x4080, 0x3C00), (0x7F7F, 0x7F7F), (0xFF7F, 0xFF7F),
        (0x7F7F, 0x7B80), (0x0001, 0x0001), (0x0001, 0x8001), (0x8000, 0x8000),
        (0x0080, 0x8001), (0x007F, 0x0001), (0x3F80, 0xBF80), (0x4B00, 0x3F00),
    ]
    nan_pairs = [(0x7FA1, 0x3F80), (0xFFA1, 0x3F80), (0x7FC5, 0x0000), (0x3F80, 0xFFB3)]
    cols = 64
    Mb = np.zeros((1, 2, cols), dtype=np.uint16)
    Gb = np.zeros((1, 2, cols), dtype=np.uint16)
    for j, (m, g) in enumerate(pairs):
        Mb[0, 0, j], Gb[0, 0, j] = m, g
    for j, (m, g) in enumerate(nan_pairs):
        Mb[0, 1, j], Gb[0, 1, j] = m, g
    M = torch.from_numpy(Mb.view(np.int16)).view(torch.bfloat16).to(DEV)
    G = torch.from_numpy(Gb.view(np.int16)).view(torch.bfloat16).to(DEV)
    Mh, Gh = to64(M), to64(G)
    idx = torch.empty(1, 1, dtype=torch.int32, device=DEV)
    d.dion3_momentum_rowsel(M, G, 1, idx)
    torch.cuda.synchronize()
    out = bits(M)[0].astype(np.uint16)
    ref = np_bits(O.momentum_accumulate(Mh[0, 0:1], Gh[0, 0:1], "bf16"), torch.bfloat16).astype(np.uint16)
    assert np.array_equal(out[0, :len(pairs)], ref[0, :len(pairs)]), (out[0, :len(pairs)], ref[0, :len(pairs)])
    for j, (m, g) in enumerate(nan_pairs):
        v = int(out[1, j])
        print(f"NaN case {m:#06x} + {g:#06x} -> {v:#06x}")
        nan_in = m if (m & 0x7FFF) > 0x7F80 else g
        assert v == (nan_in | 0x0040), (hex(m), hex(g), hex(v))


def test_rowsel_ties_and_nan(d):
    rows, cols = 40, 96
    g = torch.zeros(1, rows, cols, dtype=torch.float32)
    rng = np.random.default_rng(3)
    base = rng.standard_normal(cols).astype(np.float32)
    for r in [5, 9, 17, 30]:
        g[0, r] = torch.from_numpy(base)           # four identical rows (equal keys)
    g[0, 2] = torch.from_numpy(base * 0.5)
    g[0, 33, 7] = float("nan")
    G = g.to(DEV)
    M0 = torch.zeros_like(G)
    for k, want in [(1, [33]), (3, [5, 9, 33]), (5, [5, 9, 17, 30, 33]), (6, [2, 5, 9, 17, 30, 33]),
                    (8, [0, 1, 2, 5, 9, 17, 30, 33])]:
        _, _, _, idx, _, _, _ = _rowsel_case(d, rows, cols, 1, "f32", k, G=G, M0=M0)
        assert list(idx[0]) == want, (k, idx[0])


def test_rowsel_deterministic(d):
    outs = []
    for _ in range(2):
        M, _, _, idx, keys, sqn, _ = _rowsel_case(d, 700, 300, 2, "bf16", 75)
        outs.append((bits(M), idx, keys.view(np.int64), sqn.view(np.int64)))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


# ------------------------------------------------------------------- gather
@pytest.mark.parametrize("dt,xdt", [("bf16", "f16"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("rows,cols,batch,f", [(256, 1024, 1, 1.0), (300, 1000, 2, 0.25), (600, 200, 2, 0.25),
                                               (130, 77, 1, 0.5)])
def test_gather(d, dt, xdt, rows, cols, batch, f):
    n = min(rows, cols)
    k = O.k_from_fraction(n, f)
    M, Mh, Gh, idx, keys, sqn, ax = _rowsel_case(d, rows, cols, batch, dt, k)
    m = cols if ax == 0 else rows
    X = torch.empty(batch, k, m, dtype=TD[xdt], device=DEV)
    d.dion3_gather_rows(M, torch.from_numpy(idx).to(DEV), k, torch.from_numpy(sqn).to(DEV), X, eps=1e-7)
    torch.cuda.synchronize()
    for b in range(batch):
        Mc = to64(M[b]) if ax == 0 else to64(M[b]).T
        ref = O.frobenius_normalize(Mc[idx[b]], 1e-7)
        tol = 1e-3 if xdt == "f16" else 1e-6
        assert rel_fro(to64(X[b]), ref) <= tol


# -------------------------------------------------------------------- apply
@pytest.mark.parametrize("dt,odt", [("bf16", "f16"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("rows,cols,batch,f,wd", [(256, 1024, 1, 1.0, 0.0), (300, 1000, 2, 0.25, 0.0),
                                                  (600, 200, 2, 0.25, 0.0), (300, 1000, 1, 0.25, 0.1),
                                                  (600, 200, 1, 0.25, 0.1), (130, 77, 1, 0.5, 0.0)])
def test_apply_rows_bit_exact(d, dt, odt, rows, cols, batch, f, wd):
    n = min(rows, cols)
    k = O.k_from_fraction(n, f)
    ax = 0 if rows <= cols else 1
    m = cols if ax == 0 else rows
    W = synth.weights(rows, cols, batch, dtype=dt, device=DEV, group_seed=2)
    M = synth.gradient(rows, cols, batch, dtype=dt, device=DEV, group_seed=5)
    Ov = synth.dense(k, m, batch, dtype=odt, device=DEV, seed=9, std=0.03)
    rng = np.random.default_rng(rows)
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(batch)]).astype(np.int32)
    Wh, Mh, Oh = to64(W), to64(M), to64(Ov)
    eta, mu = 0.04, 0.95
    d.dion3_apply_rows(W, M, torch.from_numpy(idx).to(DEV), k, Ov, eta, wd, mu)
    torch.cuda.synchronize()
    for b in range(batch):
        Wc, Mc = (Wh[b], Mh[b]) if ax == 0 else (Wh[b].T, Mh[b].T)
        Wr, Mr = O.apply_rows(Wc, Mc, idx[b], Oh[b], eta, wd, mu, dt)
        if ax == 1:
            Wr, Mr = Wr.T, Mr.T
        assert np.array_equal(bits(W[b]), np_bits(Wr, TD[dt]))
        assert np.array_equal(bits(M[b]), np_bits(Mr, TD[dt]))


# ------------------------------------------------------- Gram Newton-Schulz
@pytest.mark.parametrize("xdt,tol", [("f32", 1e-4), ("f16", 3e-2)])
@pytest.mark.parametrize("b,k,m", [(1, 256, 1024), (2, 128, 512), (2, 100, 300), (1, 64, 64)])
def test_gram_ns(d, xdt, tol, b, k, m):
    rng = np.random.default_rng(k + m)
    X = rng.standard_normal((b, k, m)) * np.exp(rng.standard_normal((b, k, 1)))
    X0 = np.stack([O.frobenius_normalize(x, 1e-7) for x in X])
    Xd = torch.from_numpy(X0).to(TD[xdt]).to(DEV)
    Od = torch.empty_like(Xd)
    params = d.make_ns_params(ns_dtype=d.dtype_code(TD[xdt]))
    d.dion3_gram_ns_gathered(Xd, Od, params)
    torch.cuda.synchronize()
    xin = to64(Xd)
    for i in range(b):
        ref = O.ns_gram(xin[i], eps=0.0)   # input already normalised (up to its rounding)
        err = rel_fro(to64(Od[i]), ref)
        assert err <= tol, err
        if xdt == "f16":
            assert err <= 1e-2   # the fp16 storage model predicts about 1e-3


@pytest.mark.parametrize("dt,xdt,tol", [("bf16", "f16", 3e-2), ("f32", "f32", 1e-4), ("bf16", "f32", 1e-4)])
@pytest.mark.parametrize("rows,cols,batch,f", [(300, 1000, 2, 0.25), (600, 200, 2, 0.25), (256, 1024, 1, 1.0),
                                               (1100, 520, 1, 0.5)])
def test_gram_ns_group_form(d, dt, xdt, tol, rows, cols, batch, f):
    """dion3_gram_ns in its (group, M, idx, k) form: the selected submatrix is
    normalised and orthogonalised like the oracle's step (Section 2, Section
    4), and agrees with momentum_rowsel + gather + the gathered form."""
    n = min(rows, cols)
    k = O.k_from_fraction(n, f)
    M, Mh, Gh, idx, keys, sqn, ax = _rowsel_case(d, rows, cols, batch, dt, k)
    m = cols if ax == 0 else rows
    idx_d = torch.from_numpy(idx).to(DEV)
    params = d.make_ns_params(ns_dtype=d.dtype_code(TD[xdt]))
    Og = torch.empty(batch, k, m, dtype=TD[xdt], device=DEV)
    d.dion3_gram_ns(M, idx_d, k, Og, params)
    X = torch.empty(batch, k, m, dtype=TD[xdt], device=DEV)
    Ox = torch.empty_like(X)
    d.dion3_gather_rows(M, idx_d, k, torch.from_numpy(sqn).to(DEV), X, eps=params.eps)
    d.dion3_gram_ns_gathered(X, Ox, params)
    torch.cuda.synchronize()
    for b in range(batch):
        Mc = to64(M[b]) if ax == 0 else to64(M[b]).T
        ref = O.ns_gram(Mc[idx[b]])
        assert rel_fro(to64(Og[b]), ref) <= tol
        # same normalised input up to the last bit of the fp64 norm: the two
        # forms agree far inside the tolerance
        assert rel_fro(to64(Og[b]), to64(Ox[b])) <= (2e-3 if xdt == "f16" else 1e-6)


def test_gram_ns_group_form_zero_selection(d):
    """An all-zero selected submatrix gives O = 0 (the eps guard of the
    normalisation)."""
    M = torch.zeros(2, 64, 200, dtype=torch.bfloat16, device=DEV)
    idx = torch.arange(16, dtype=torch.int32, device=DEV).repeat(2, 1)
    Og = torch.full((2, 16, 200), 7.0, dtype=torch.float16, device=DEV)
    d.dion3_gram_ns(M, idx, 16, Og, d.make_ns_params(ns_dtype=d.F16))
    torch.cuda.synchronize()
    assert torch.count_nonzero(Og).item() == 0


def test_gram_ns_restart_variants(d):
    b, k, m = 1, 128, 512
    rng = np.random.default_rng(1)
    X0 = O.frobenius_normalize(rng.standard_normal((k, m)) * np.exp(rng.standard_normal((k, 1))))
    Xd = torch.from_numpy(X0[None]).float().to(DEV)
    for mask, restart in [(0, ()), (1 << 2, (2,)), ((1 << 1) | (1 << 3), (1, 3)), ((1 << 1) | (1 << 2) | (1 << 3) | (1 << 4), (1, 2, 3, 4))]:
        Od = torch.empty_like(Xd)
        d.dion3_gram_ns_gathered(Xd, Od, d.make_ns_params(restart_mask=mask, ns_dtype=d.F32))
        torch.cuda.synchronize()
        ref = O.ns_gram(to64(Xd)[0], restart_after=restart, eps=0.0)
        assert rel_fro(to64(Od)[0], ref) <= 1e-4, mask


# ---------------------------------------------------- standard Newton-Schulz
@pytest.mark.parametrize("xdt,tol", [("f32", 1e-4), ("f16", 3e-2)])
@pytest.mark.parametrize("b,k,m", [(2, 128, 512), (2, 100, 300), (1, 256, 256), (1, 64, 64)])
def test_standard_ns(d, xdt, tol, b, k, m):
    """dion3_standard_ns against the oracle's standard Newton-Schulz."""
    rng = np.random.default_rng(3 * k + m)
    X = rng.standard_normal((b, k, m)) * np.exp(rng.standard_normal((b, k, 1)))
    X0 = np.stack([O.frobenius_normalize(x, 1e-7) for x in X])
    Xd = torch.from_numpy(X0).to(TD[xdt]).to(DEV)
    Od = torch.empty_like(Xd)
    d.dion3_standard_ns(Xd, Od, d.make_ns_params(ns_dtype=d.dtype_code(TD[xdt])))
    torch.cuda.synchronize()
    xin = to64(Xd)
    for i in range(b):
        err = rel_fro(to64(Od[i]), O.ns_standard(xin[i], eps=0.0))
        assert err <= tol, err


def test_standard_ns_large_tiles(d):
    """52 square 1024 x 1024 inputs: every product runs on the 256 x 256 kernels
    (520 symmetric tiles, 832 rectangular tiles); first and last checked."""
    b, k = 52, 1024
    Xd = synth.dense(k, k, b, dtype="f16", device=DEV, seed=5)
    Xd = (Xd.float() / Xd.float().flatten(1).norm(dim=1).view(b, 1, 1)).half()
    Od = torch.empty_like(Xd)
    d.dion3_standard_ns(Xd, Od, d.make_ns_params(ns_dtype=d.F16))
    torch.cuda.synchronize()
    for i in (0, b - 1):
        err = rel_fro(to64(Od[i]), O.ns_standard(to64(Xd[i]), eps=0.0))
        assert err <= 3e-2, (i, err)


def test_gemm_deterministic(d):
    A = synth.dense(512, 1024, 2, dtype="f16", device=DEV, seed=1)
    outs = []
    for _ in range(2):
        C = torch.empty(2, 512, 512, dtype=torch.float16, device=DEV)
        d.dion3_syrk(A, C)
        torch.cuda.synchronize()
        outs.append(bits(C))
    assert np.array_equal(outs[0], outs[1])


# ---------------------------------------------- large-tile launch configuration
# Batched shapes of the Newton-Schulz products at the sizes the step uses
# (k = 1024 and 1280 selected lines, m up to 11008), large enough that the
# library takes its 256 x 256 tile.  Every matrix is checked for exact
# symmetry; a sample of matrices is compared with fp64 products.  (The
# library picks the large tile when a launch has at least 128 of them.)
def _sample(b):
    return sorted({0, b // 2, b - 1})


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("b,n,kd", [(52, 1024, 1024), (52, 1024, 11008), (36, 1280, 1280)])
def test_syrk_large_tiles(d, dt, b, n, kd):
    A = synth.dense(n, kd, b, dtype=dt, device=DEV, seed=n + kd + b)
    C = torch.full((b, n, n), float("nan"), dtype=TD[dt], device=DEV)
    d.dion3_syrk(A, C)
    torch.cuda.synchronize()
    cb = bits(C)
    assert np.array_equal(cb, cb.transpose(0, 2, 1))
    for i in _sample(b):
        a = to64(A[i])
        got = to64(C[i])
        assert np.all(np.isfinite(got))
        assert rel_fro(got, a @ a.T) <= TOL[dt], i


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("b,n", [(52, 1024), (36, 1280)])
def test_sym_products_large_tiles(d, dt, b, n):
    A = synth.symmetric(n, b, dtype=dt, device=DEV, seed=31)
    B = synth.symmetric(n, b, dtype=dt, device=DEV, seed=32)
    C = torch.empty_like(A)
    al, be, ga = 2.0315, -4.7750, 3.4445
    d.dion3_sym_sq_add(A, B, C, alpha=al, beta=be, gamma=ga)
    torch.cuda.synchronize()
    cb = bits(C)
    assert np.array_equal(cb, cb.transpose(0, 2, 1))
    for i in _sample(b):
        a, bb = to64(A[i]), to64(B[i])
        assert rel_fro(to64(C[i]), al * a @ a + be * bb + ga * np.eye(n)) <= TOL[dt], i
    # product of two commuting polynomials of one symmetric matrix
    S = A
    P = torch.empty_like(A)
    d.dion3_sym_sq_add(S, S, P, alpha=0.4, beta=-0.2, gamma=0.3)   # P = 0.4 S^2 - 0.2 S + 0.3 I
    C2 = torch.empty_like(A)
    d.dion3_sym_mul(S, P, C2, alpha=1.0)
    torch.cuda.synchronize()
    cb = bits(C2)
    assert np.array_equal(cb, cb.transpose(0, 2, 1))
    for i in _sample(b):
        ref = to64(S[i]) @ to64(P[i])
        ref = np.tril(ref) + np.tril(ref, -1).T
        assert rel_fro(to64(C2[i]), ref) <= TOL[dt], i


@pytest.mark.parametrize("dt,odt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "f32")])
@pytest.mark.parametrize("b,k,m", [(8, 1024, 4096), (3, 1024, 11008), (6, 1280, 5120)])
def test_gemm_qx_large_tiles(d, dt, odt, b, k, m):
    Q = synth.symmetric(k, b, dtype=dt, device=DEV, seed=k + b)
    X = synth.dense(k, m, b, dtype=dt, device=DEV, seed=m + b)
    Y = torch.empty(b, k, m, dtype=TD[odt], device=DEV)
    d.dion3_gemm(Q, X, Y, alpha=1.0)
    torch.cuda.synchronize()
    for i in _sample(b):
        ref = to64(Q[i]) @ to64(X[i])
        assert rel_fro(to64(Y[i]), ref) <= TOL[odt if odt != "f32" else dt], i


def test_products_independent_of_batch(d):
    """Each matrix's product is the same bits whether it runs alone (128 x 128
    tiles: too few tiles for the large kernel) or in a batch large enough for
    the 256 x 256 tiles, so splitting a Newton-Schulz batch does not change
    any result."""
    g = torch.Generator(device="cpu").manual_seed(7)
    n, m, b = 1024, 512, 16
    X = (torch.randn(b, n, m, generator=g) / m ** 0.5).to(torch.float16).to(DEV)
    Q = (torch.randn(b, n, n, generator=g) / n ** 0.5).to(torch.float16).to(DEV)
    E = (torch.randn(b, n, n, generator=g) / n ** 0.5).to(torch.float16).to(DEV)
    E = ((E + E.transpose(1, 2)) * 0.5).contiguous()
    full = torch.empty(b, n, n, dtype=torch.float16, device=DEV)
    one = torch.empty(1, n, n, dtype=torch.float16, device=DEV)
    d.dion3_syrk(X, full, 0.5, 0.0)
    d.dion3_syrk(X[3:4], one, 0.5, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(full[3].view(torch.int16), one[0].view(torch.int16)), "syrk"
    d.dion3_sym_sq_add(E, E, full, -0.25, 0.75, 1.5)
    d.dion3_sym_sq_add(E[3:4], E[3:4], one, -0.25, 0.75, 1.5)
    torch.cuda.synchronize()
    assert torch.equal(full[3].view(torch.int16), one[0].view(torch.int16)), "sym_sq_add"
    Y = torch.empty(b, n, m, dtype=torch.float16, device=DEV)
    Y1 = torch.empty(1, n, m, dtype=torch.float16, device=DEV)
    d.dion3_gemm(Q, X, Y, 1.0)
    d.dion3_gemm(Q[3:4], X[3:4], Y1, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(Y[3].view(torch.int16), Y1[0].view(torch.int16)), "gemm"


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_multi_tile_products_match_single_matrices(d, dt):
    """Batches large enough for work-groups that run several 256 x 256 tiles
    back to back (diagonal and off-diagonal tiles of different matrices in
    one work-group, one-panel diagonal tiles of X X^T and A^2 + B among them)
    against every matrix computed alone, where the 128 x 128 kernel runs it:
    the same bits for every matrix."""
    g = torch.Generator(device="cpu").manual_seed(19)
    t = TD[dt]
    n, m, b = 1024, 2048, 48
    X = (torch.randn(b, n, m, generator=g) / m ** 0.5).to(t).to(DEV)
    A = (torch.randn(b, n, n, generator=g) / n ** 0.5)
    A = ((A + A.transpose(1, 2)) * 0.5).to(t).to(DEV).contiguous()
    B = (torch.randn(b, n, n, generator=g) / n ** 0.5)
    B = ((B + B.transpose(1, 2)) * 0.5).to(t).to(DEV).contiguous()
    one = torch.empty(1, n, n, dtype=t, device=DEV)
    onex = torch.empty(1, n, m, dtype=t, device=DEV)
    cases = [
        ("syrk", lambda out, sl: d.dion3_syrk(X[sl], out, 1.0, 0.0), (n, n)),
        ("sym_sq_add", lambda out, sl: d.dion3_sym_sq_add(A[sl], B[sl], out, 0.5, -1.25, 2.0), (n, n)),
        ("sym_mul", lambda out, sl: d.dion3_sym_mul(A[sl], B[sl], out, 1.0), (n, n)),
        ("gemm", lambda out, sl: d.dion3_gemm(A[sl], X[sl], out, 1.0), (n, m)),
    ]
    for name, run, shape in cases:
        full = torch.empty(b, *shape, dtype=t, device=DEV)
        run(full, slice(0, b))
        torch.cuda.synchronize()
        for i in range(b):
            single = one if shape == (n, n) else onex
            run(single, slice(i, i + 1))
            torch.cuda.synchronize()
            assert torch.equal(full[i].view(torch.int16), single[0].view(torch.int16)), (name, i)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_count_nonfinite(d, dt):
    """dion3_count_nonfinite counts NaN and +-Inf entries exactly: planted at
    random positions of ragged sizes, on aligned and misaligned starts
    (vector and scalar paths), against torch.isfinite; finite extremes (the
    largest finite value, subnormals) are not counted."""
    g = torch.Generator().manual_seed(11)
    big = torch.finfo(TD[dt]).max
    for n in [1, 7, 1000, (1 << 20) + 3]:
        x = torch.randn(n + 1, generator=g).to(TD[dt])
        x[torch.randint(0, n + 1, (max(1, n // 97),), generator=g)] = float("nan")
        x[torch.randint(0, n + 1, (max(1, n // 131),), generator=g)] = float("inf")
        x[torch.randint(0, n + 1, (max(1, n // 173),), generator=g)] = float("-inf")
        x[torch.randint(0, n + 1, (max(1, n // 191),), generator=g)] = big
        x[torch.randint(0, n + 1, (max(1, n // 211),), generator=g)] = torch.finfo(TD[dt]).tiny / 4
        xd = x.to(DEV)
        for view in (xd[:n], xd[1:]):          # 16-byte aligned start, then a misaligned one
            want = int((~torch.isfinite(view.cpu().float())).sum())
            assert d.dion3_count_nonfinite(view.contiguous() if not view.is_contiguous() else view) == want, (n, want)
        # accumulation into a caller counter across two calls
        cnt = torch.zeros(1, dtype=torch.int64, device=DEV)
        d.dion3_count_nonfinite(xd[:n], cnt)
        d.dion3_count_nonfinite(xd[1:], cnt)
        torch.cuda.synchronize()
        assert int(cnt.item()) == int((~torch.isfinite(x[:n].float())).sum()) + int((~torch.isfinite(x[1:].float())).sum())
