"""ctypes binding of libdion3.so: the C entry points under the same names.

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the optimizer runs in the library's kernels.
Importing this module raises if the library has not been built, so a missing
extension can never fall back to anything else.
"""

from __future__ import annotations

import atexit
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DION3_LIB names another build of the same library (the host sanitizer build
# of the CPU tests); by default the in-tree libdion3.so
LIB_PATH = os.environ.get("DION3_LIB") or os.path.join(_HERE, "libdion3.so")

F32, F16, BF16 = 0, 1, 2
GRAPH_ONE = 1                    # DION3_GRAPH_ONE
_TORCH_TO_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_DT_TO_TORCH = {v: k for k, v in _TORCH_TO_DT.items()}

# Muon's published fixed quintic (a, b, c), used for every iteration unless a
# table is given ("Dion3: Full-Stack Orthogonal Updates", Section 2 names the
# coefficient sources but prints no values).
DEFAULT_QUINTIC = (3.4445, -4.7750, 2.0315)
DEFAULT_T = 5
DEFAULT_RESTART_MASK = 1 << 2      # restart after iteration 2 (Section 4)
DEFAULT_EPS = 1e-7


class Dion3Error(RuntimeError):
    pass


class Group(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int), ("cols", ctypes.c_int), ("batch", ctypes.c_int),
                ("batch_stride", ctypes.c_longlong), ("dtype", ctypes.c_int),
                ("sel_axis", ctypes.c_int)]


class NSParams(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int), ("coeffs", ctypes.POINTER(ctypes.c_double)),
                ("restart_mask", ctypes.c_uint), ("eps", ctypes.c_float), ("ns_dtype", ctypes.c_int)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, ll, f, d, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float,
                           ctypes.c_double, ctypes.c_size_t)
    gp = ctypes.POINTER(Group)
    pp = ctypes.POINTER(NSParams)
    sig = {
        "dion3_k_from_fraction": (i, [i, d]),
        "dion3_canonical": (i, [gp, ctypes.POINTER(i), ctypes.POINTER(i), ctypes.POINTER(i)]),
        "dion3_status_string": (ctypes.c_char_p, [i]),
        "dion3_rowsel_workspace_bytes": (sz, [gp]),
        "dion3_momentum_rowsel": (i, [gp, vp, vp, i, vp, vp, vp, vp, sz, vp]),
        "dion3_momentum_rowsel_ef": (i, [gp, vp, vp, i, vp, vp, vp, vp, i, f, vp, sz, vp]),
        "dion3_decay_rows": (i, [gp, vp, vp, i, f, vp]),
        "dion3_momentum_rowsel_noalloc": (i, [gp, vp, vp, i, vp, vp, vp, vp, i, f, vp]),
        "dion3_step_deferred": (i, [i, gp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                    ctypes.POINTER(i), ctypes.POINTER(vp), i, pp, f, f, f, vp, sz, vp]),
        "dion3_gather_rows": (i, [gp, vp, vp, i, vp, f, i, vp, vp]),
        "dion3_gram_ns_gathered_workspace_bytes": (sz, [i, i, i, i]),
        "dion3_gram_ns_gathered": (i, [i, i, i, pp, vp, vp, vp, sz, vp]),
        "dion3_gram_ns_workspace_bytes": (sz, [gp, i, pp]),
        "dion3_workspace_bytes": (sz, [gp, i, pp]),
        "dion3_gram_ns": (i, [gp, vp, vp, i, pp, vp, vp, sz, vp]),
        "dion3_release": (i, []),
        "dion3_standard_ns_workspace_bytes": (sz, [i, i, i, i]),
        "dion3_standard_ns": (i, [i, i, i, pp, vp, vp, vp, sz, vp]),
        "dion3_syrk": (i, [i, i, i, i, vp, ll, vp, ll, f, f, vp]),
        "dion3_sym_sq_add": (i, [i, i, i, vp, ll, vp, ll, vp, ll, f, f, f, vp]),
        "dion3_sym_mul": (i, [i, i, i, vp, ll, vp, ll, vp, ll, f, vp]),
        "dion3_gemm": (i, [i, i, i, i, vp, ll, vp, ll, i, vp, ll, f, vp]),
        "dion3_apply_rows": (i, [gp, vp, vp, vp, i, vp, i, ll, f, f, f, vp]),
        "dion3_apply_rows_scaled": (i, [gp, vp, vp, vp, i, vp, i, ll, vp, f, f, f, vp]),
        "dion3_normuon_scale": (i, [gp, vp, i, vp, i, ll, vp, f, f, vp, vp]),
        "dion3_step_normuon": (i, [i, gp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                   ctypes.POINTER(i), ctypes.POINTER(vp), ctypes.POINTER(vp), i, i, pp,
                                   f, f, f, f, f, vp, sz, vp]),
        "dion3_step_workspace_bytes": (sz, [i, gp, ctypes.POINTER(i), pp]),
        "dion3_step": (i, [i, gp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                           ctypes.POINTER(i), ctypes.POINTER(vp), pp, f, f, f, vp, sz, vp]),
        "dion3_step_graph_create": (i, [i, gp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                        ctypes.POINTER(i), ctypes.POINTER(vp), i, pp, f, f, f, vp, sz,
                                        ctypes.c_uint, ctypes.POINTER(vp)]),
        "dion3_step_normuon_graph_create": (i, [i, gp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                                ctypes.POINTER(vp), ctypes.POINTER(i), ctypes.POINTER(vp),
                                                ctypes.POINTER(vp), i, pp, f, f, f, f, f, vp, sz,
                                                ctypes.c_uint, ctypes.POINTER(vp)]),
        "dion3_graph_launch": (i, [vp, vp]),
        "dion3_count_nonfinite": (i, [vp, i, sz, vp, vp]),
        "dion3_graph_destroy": (i, [vp]),
        "dion3_timing_enable": (i, [i]),
        "dion3_timing_report": (i, [ctypes.c_char_p, sz]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()
# the library's own streams and events go before the HIP runtime shuts down
atexit.register(lib.dion3_release)


# ------------------------------------------------------------------ helpers
def _check(status: int, what: str) -> None:
    if status < 0:
        raise Dion3Error(f"{what}: {lib.dion3_status_string(status).decode()} ({status})")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise Dion3Error("tensor must live on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def dtype_code(dt: torch.dtype) -> int:
    return _TORCH_TO_DT[dt]


def torch_dtype(code: int) -> torch.dtype:
    return _DT_TO_TORCH[code]


def make_group(t: torch.Tensor, sel_axis: int = -1) -> Group:
    """Describe a [batch, rows, cols] tensor (rows and cols contiguous)."""
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise Dion3Error("group tensor must be [batch, rows, cols] with packed rows")
    return Group(t.shape[1], t.shape[2], t.shape[0], t.stride(0), dtype_code(t.dtype), sel_axis)


def make_ns_params(coeffs=None, T: int = DEFAULT_T, restart_mask: int = DEFAULT_RESTART_MASK,
                   eps: float = DEFAULT_EPS, ns_dtype: int = F16):
    """NSParams plus the ctypes array that keeps its coefficient table alive."""
    if coeffs is None:
        coeffs = [DEFAULT_QUINTIC] * T
    flat = [float(v) for row in coeffs for v in row]
    arr = (ctypes.c_double * len(flat))(*flat)
    p = NSParams(len(coeffs), ctypes.cast(arr, ctypes.POINTER(ctypes.c_double)), restart_mask, eps, ns_dtype)
    p._keep = arr
    return p


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# -------------------------------------------------------------- entry points
def dion3_k_from_fraction(n: int, f: float) -> int:
    k = lib.dion3_k_from_fraction(n, f)
    _check(k, "dion3_k_from_fraction")
    return k


def dion3_canonical(g: Group):
    n, m, a = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib.dion3_canonical(ctypes.byref(g), ctypes.byref(n), ctypes.byref(m), ctypes.byref(a)),
           "dion3_canonical")
    return n.value, m.value, a.value


def dion3_rowsel_workspace_bytes(g: Group) -> int:
    return lib.dion3_rowsel_workspace_bytes(ctypes.byref(g))


def dion3_momentum_rowsel(M, G, k, idx, keys=None, sel_sqnorm=None, ws=None, sel_axis=-1):
    g = make_group(M, sel_axis)
    if ws is None:
        ws = workspace(dion3_rowsel_workspace_bytes(g), M.device)
    _check(lib.dion3_momentum_rowsel(ctypes.byref(g), _ptr(M), _ptr(G), k, _ptr(idx), _ptr(keys),
                                     _ptr(sel_sqnorm), _ptr(ws), ws.numel(), _stream()),
           "dion3_momentum_rowsel")


def dion3_momentum_rowsel_ef(M, G, k, idx, prev_idx, prev_k, mu, keys=None, sel_sqnorm=None, ws=None,
                             sel_axis=-1):
    g = make_group(M, sel_axis)
    if ws is None:
        ws = workspace(dion3_rowsel_workspace_bytes(g), M.device)
    _check(lib.dion3_momentum_rowsel_ef(ctypes.byref(g), _ptr(M), _ptr(G), k, _ptr(idx), _ptr(keys),
                                        _ptr(sel_sqnorm), _ptr(prev_idx), prev_k, mu, _ptr(ws), ws.numel(),
                                        _stream()), "dion3_momentum_rowsel_ef")


def dion3_momentum_rowsel_noalloc(M, G, k, idx, keys=None, sel_sqnorm=None, prev_idx=None, prev_k=0, mu=0.0,
                                  sel_axis=-1):
    """dion3_momentum_rowsel_ef with the library's fixed per-GPU scratch
    instead of a workspace (no allocation, no workspace argument)."""
    g = make_group(M, sel_axis)
    _check(lib.dion3_momentum_rowsel_noalloc(ctypes.byref(g), _ptr(M), _ptr(G), k, _ptr(idx), _ptr(keys),
                                             _ptr(sel_sqnorm), _ptr(prev_idx), prev_k, mu, _stream()),
           "dion3_momentum_rowsel_noalloc")


def dion3_decay_rows(M, idx, k, mu, sel_axis=-1):
    g = make_group(M, sel_axis)
    _check(lib.dion3_decay_rows(ctypes.byref(g), _ptr(M), _ptr(idx), k, mu, _stream()), "dion3_decay_rows")


def dion3_gather_rows(M, idx, k, sel_sqnorm, X, eps=DEFAULT_EPS, sel_axis=-1):
    g = make_group(M, sel_axis)
    _check(lib.dion3_gather_rows(ctypes.byref(g), _ptr(M), _ptr(idx), k, _ptr(sel_sqnorm), eps,
                                 dtype_code(X.dtype), _ptr(X), _stream()), "dion3_gather_rows")


def dion3_gram_ns_gathered_workspace_bytes(batch, k, m, ns_dtype) -> int:
    return lib.dion3_gram_ns_gathered_workspace_bytes(batch, k, m, ns_dtype)


def dion3_gram_ns_gathered(X0, O, params=None, ws=None):
    b, k, m = X0.shape
    p = params if params is not None else make_ns_params(ns_dtype=dtype_code(X0.dtype))
    if ws is None:
        ws = workspace(dion3_gram_ns_gathered_workspace_bytes(b, k, m, p.ns_dtype), X0.device)
    _check(lib.dion3_gram_ns_gathered(b, k, m, ctypes.byref(p), _ptr(X0), _ptr(O), _ptr(ws), ws.numel(),
                                      _stream()), "dion3_gram_ns_gathered")


def dion3_gram_ns_workspace_bytes(g: Group, k: int, params) -> int:
    return lib.dion3_gram_ns_workspace_bytes(ctypes.byref(g), k, ctypes.byref(params))


def dion3_workspace_bytes(g: Group, k: int, params) -> int:
    return lib.dion3_workspace_bytes(ctypes.byref(g), k, ctypes.byref(params))


def dion3_gram_ns(M, idx, k, O, params=None, ws=None, sel_axis=-1):
    """Gram Newton-Schulz of the selected submatrices M[b][idx[b], :] of the
    group tensor M (canonical orientation) into O [batch][k][m]."""
    g = make_group(M, sel_axis)
    p = params if params is not None else make_ns_params(ns_dtype=dtype_code(O.dtype))
    if ws is None:
        nb = dion3_gram_ns_workspace_bytes(g, k, p)
        if nb == 0:
            raise Dion3Error("dion3_gram_ns_workspace_bytes: invalid arguments")
        ws = workspace(nb, M.device)
    _check(lib.dion3_gram_ns(ctypes.byref(g), _ptr(M), _ptr(idx), k, ctypes.byref(p), _ptr(O), _ptr(ws),
                             ws.numel(), _stream()), "dion3_gram_ns")


def dion3_release() -> None:
    """Destroy the library's own streams, events and timing events."""
    _check(lib.dion3_release(), "dion3_release")


def dion3_standard_ns_workspace_bytes(batch, k, m, ns_dtype) -> int:
    return lib.dion3_standard_ns_workspace_bytes(batch, k, m, ns_dtype)


def dion3_standard_ns(X0, O, params=None, ws=None):
    b, k, m = X0.shape
    p = params if params is not None else make_ns_params(ns_dtype=dtype_code(X0.dtype))
    if ws is None:
        ws = workspace(dion3_standard_ns_workspace_bytes(b, k, m, p.ns_dtype), X0.device)
    _check(lib.dion3_standard_ns(b, k, m, ctypes.byref(p), _ptr(X0), _ptr(O), _ptr(ws), ws.numel(),
                                 _stream()), "dion3_standard_ns")


def dion3_syrk(A, C, alpha=1.0, beta=0.0):
    b, n, kd = A.shape
    _check(lib.dion3_syrk(b, n, kd, dtype_code(A.dtype), _ptr(A), A.stride(0), _ptr(C), C.stride(0),
                          alpha, beta, _stream()), "dion3_syrk")


def dion3_sym_sq_add(A, B, C, alpha=1.0, beta=1.0, gamma=0.0):
    b, n, _ = A.shape
    _check(lib.dion3_sym_sq_add(b, n, dtype_code(A.dtype), _ptr(A), A.stride(0), _ptr(B), B.stride(0),
                                _ptr(C), C.stride(0), alpha, beta, gamma, _stream()), "dion3_sym_sq_add")


def dion3_sym_mul(A, B, C, alpha=1.0):
    b, n, _ = A.shape
    _check(lib.dion3_sym_mul(b, n, dtype_code(A.dtype), _ptr(A), A.stride(0), _ptr(B), B.stride(0),
                             _ptr(C), C.stride(0), alpha, _stream()), "dion3_sym_mul")


def dion3_gemm(Q, X, Y, alpha=1.0):
    b, k, m = X.shape
    _check(lib.dion3_gemm(b, k, m, dtype_code(Q.dtype), _ptr(Q), Q.stride(0), _ptr(X), X.stride(0),
                          dtype_code(Y.dtype), _ptr(Y), Y.stride(0), alpha, _stream()), "dion3_gemm")


def dion3_apply_rows(W, M, idx, k, O, eta, wd, mu, sel_axis=-1):
    g = make_group(W, sel_axis)
    _check(lib.dion3_apply_rows(ctypes.byref(g), _ptr(W), _ptr(M), _ptr(idx), k, _ptr(O),
                                dtype_code(O.dtype), O.stride(0), eta, wd, mu, _stream()),
           "dion3_apply_rows")


def dion3_normuon_scale(M, idx, k, O, V, row_scale, beta2=0.95, eps=1e-8, sel_axis=-1):
    """NorMuon row factors of the canonical Newton-Schulz output O [batch][k][m]
    of the group whose tensor is M; V [batch][n] fp32 is updated in place."""
    g = make_group(M, sel_axis)
    _check(lib.dion3_normuon_scale(ctypes.byref(g), _ptr(idx), k, _ptr(O), dtype_code(O.dtype),
                                   O.stride(0), _ptr(V), beta2, eps, _ptr(row_scale), _stream()),
           "dion3_normuon_scale")


def dion3_apply_rows_scaled(W, M, idx, k, O, row_scale, eta, wd, mu, sel_axis=-1):
    g = make_group(W, sel_axis)
    _check(lib.dion3_apply_rows_scaled(ctypes.byref(g), _ptr(W), _ptr(M) if M is not None else None,
                                       _ptr(idx), k, _ptr(O), dtype_code(O.dtype), O.stride(0),
                                       _ptr(row_scale) if row_scale is not None else None,
                                       eta, wd, mu, _stream()), "dion3_apply_rows_scaled")


class StepPlan:
    """Marshalled arguments of dion3_step for a fixed list of group tensors."""

    def __init__(self, Ws, Ms, Gs, ks, idxs, params, sel_axes=None):
        n = len(Ws)
        sel_axes = sel_axes or [-1] * n
        self.groups = (Group * n)(*[make_group(W, a) for W, a in zip(Ws, sel_axes)])
        self.W = (ctypes.c_void_p * n)(*[W.data_ptr() for W in Ws])
        self.M = (ctypes.c_void_p * n)(*[M.data_ptr() for M in Ms])
        self.G = (ctypes.c_void_p * n)(*[G.data_ptr() for G in Gs])
        self.k = (ctypes.c_int * n)(*ks)
        self.idx = (ctypes.c_void_p * n)(*[t.data_ptr() for t in idxs])
        self.params = params
        self.n = n
        self._keep = (Ws, Ms, Gs, idxs)
        nbytes = lib.dion3_step_workspace_bytes(n, self.groups, self.k, ctypes.byref(params))
        if nbytes == 0:
            raise Dion3Error("dion3_step_workspace_bytes: invalid groups")
        self.ws = workspace(nbytes, Ws[0].device)

    def step(self, eta, wd, mu):
        _check(lib.dion3_step(self.n, self.groups, self.W, self.M, self.G, self.k, self.idx,
                              ctypes.byref(self.params), eta, wd, mu, _ptr(self.ws), self.ws.numel(),
                              _stream()), "dion3_step")

    def step_deferred(self, eta, wd, mu, has_prev):
        """dion3_step_deferred: the idx tensors carry the previous selection in
        (has_prev) and this step's selection out; M owes its decay until the
        next step or flush_decay()."""
        _check(lib.dion3_step_deferred(self.n, self.groups, self.W, self.M, self.G, self.k, self.idx,
                                       1 if has_prev else 0, ctypes.byref(self.params), eta, wd, mu,
                                       _ptr(self.ws), self.ws.numel(), _stream()), "dion3_step_deferred")

    def step_normuon(self, Vs, eta, wd, mu, beta2=0.95, nm_eps=1e-8, deferred=False, has_prev=False):
        """dion3_step_normuon with the per-group second moments Vs ([batch][n]
        fp32 each, updated in place)."""
        V = (ctypes.c_void_p * self.n)(*[v.data_ptr() for v in Vs])
        _check(lib.dion3_step_normuon(self.n, self.groups, self.W, self.M, self.G, self.k, self.idx, V,
                                      1 if deferred else 0, 1 if has_prev else 0, ctypes.byref(self.params),
                                      eta, wd, mu, beta2, nm_eps, _ptr(self.ws), self.ws.numel(),
                                      _stream()), "dion3_step_normuon")

    def graph(self, eta, wd, mu, has_prev=True, one=False):
        """dion3_step_graph_create: the deferred step as instantiated HIP graphs
        over this plan's tensors and workspace (StepGraph); one=True builds
        the single-graph form (DION3_GRAPH_ONE)."""
        g = ctypes.c_void_p()
        _check(lib.dion3_step_graph_create(self.n, self.groups, self.W, self.M, self.G, self.k, self.idx,
                                           1 if has_prev else 0, ctypes.byref(self.params), eta, wd, mu,
                                           _ptr(self.ws), self.ws.numel(), GRAPH_ONE if one else 0,
                                           ctypes.byref(g)),
               "dion3_step_graph_create")
        return StepGraph(g, self)

    def graph_normuon(self, Vs, eta, wd, mu, beta2=0.95, nm_eps=1e-8, has_prev=True, one=False):
        """dion3_step_normuon_graph_create: the deferred NorMuon step as HIP
        graphs over this plan's tensors, workspace and the second moments Vs."""
        V = (ctypes.c_void_p * self.n)(*[v.data_ptr() for v in Vs])
        g = ctypes.c_void_p()
        _check(lib.dion3_step_normuon_graph_create(self.n, self.groups, self.W, self.M, self.G, self.k,
                                                   self.idx, V, 1 if has_prev else 0, ctypes.byref(self.params),
                                                   eta, wd, mu, beta2, nm_eps, _ptr(self.ws), self.ws.numel(),
                                                   GRAPH_ONE if one else 0, ctypes.byref(g)),
               "dion3_step_normuon_graph_create")
        return StepGraph(g, (self, Vs))

    def flush_decay(self, mu):
        """Complete the pending decay of the last deferred step on every group."""
        Ws, Ms, Gs, idxs = self._keep
        for M, idx, k, g in zip(Ms, idxs, self.k, self.groups):
            _check(lib.dion3_decay_rows(ctypes.byref(g), _ptr(M), _ptr(idx), k, mu, _stream()),
                   "dion3_decay_rows")


class StepGraph:
    """An instantiated step graph; launch() enqueues one step on the current
    stream.  Holds its plan (tensors and workspace) alive."""

    def __init__(self, handle, plan):
        self._h = handle
        self._plan = plan

    def launch(self):
        _check(lib.dion3_graph_launch(self._h, _stream()), "dion3_graph_launch")

    def destroy(self):
        if self._h:
            _check(lib.dion3_graph_destroy(self._h), "dion3_graph_destroy")
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def dion3_step(Ws, Ms, Gs, ks, idxs, eta, wd, mu, params=None, sel_axes=None):
    p = params if params is not None else make_ns_params()
    StepPlan(Ws, Ms, Gs, ks, idxs, p, sel_axes).step(eta, wd, mu)


def dion3_count_nonfinite(x, count=None) -> int:
    """Number of NaN / +-Inf entries of the device tensor x (fp32, fp16 or
    bf16).  With a caller-zeroed int64 device tensor `count` the call only
    enqueues (the library adds to it) and returns None; otherwise it uses a
    fresh counter and reads it back."""
    t = x.detach()
    if not t.is_contiguous():
        raise Dion3Error("dion3_count_nonfinite: x must be contiguous")
    own = count is None
    if own:
        count = torch.zeros(1, dtype=torch.int64, device=t.device)
    _check(lib.dion3_count_nonfinite(_ptr(t), dtype_code(t.dtype), t.numel(), _ptr(count), _stream()),
           "dion3_count_nonfinite")
    return int(count.item()) if own else None


def dion3_timing_enable(max_launches: int) -> None:
    _check(lib.dion3_timing_enable(max_launches), "dion3_timing_enable")


def dion3_timing_report() -> dict:
    buf = ctypes.create_string_buffer(1 << 16)
    nb = lib.dion3_timing_report(buf, len(buf))
    _check(nb, "dion3_timing_report")
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out
