// Host driver of Gram Newton-Schulz and the C entry points of the symmetric
// building blocks.
//
// Method: "Dion3: Full-Stack Orthogonal Updates", Section 4.  Gram
// Newton-Schulz iterates on the Gram matrix R = X X^T instead of X:
//   Z_t = a_t I + b_t R + c_t R^2        (one "A^2 + B" product)
//   Q_t = Q_{t-1} Z_t                    (free on a pass's first iteration)
//   R_t = Z_t R_{t-1} Z_t                (skipped on a pass's last iteration)
// and multiplies back once, X <- Q X, at the end of a pass.  A restart after
// iteration 2 starts a new pass on the current X (Gram matrix rebuilt, Q reset
// to the identity), which keeps spurious negative eigenvalues of R in check in
// half precision.  Every k x k product is a polynomial in the same Gram matrix,
// so it is symmetric in exact arithmetic and is computed as a lower triangle
// and mirrored (Section 5).
//
// Buffers: the k x m input X0 is read only; the pass outputs alternate between
// a k x m workspace slice and O so that the last pass writes O; four k x k
// workspace slices rotate between R, Z, Q and the Z R intermediate.
#include "common.h"

namespace dion3 {

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static int sym_op(int op, int batch, int n, int K, int dtype, const void* A, long long sA,
                  const void* B, long long sB, const void* E, long long sE, void* C, long long sC,
                  float alpha, float beta, float gamma, hipStream_t s, bool rev = false) {
  GemmArgs g;
  g.reverse = rev;
  g.op = op; g.dtype = dtype; g.out_dtype = dtype; g.batch = batch;
  g.M = n; g.N = n; g.K = K;
  g.A = A; g.lda = K; g.sA = sA;
  g.B = B; g.ldb = K; g.sB = sB;
  g.E = E; g.lde = n; g.sE = sE;
  g.C = C; g.ldc = n; g.sC = sC;
  g.alpha = alpha; g.beta = beta; g.gamma = gamma;
  return launch_gemm(g, s);
}

static int qx_op(int batch, int k, int m, int in_dtype, const void* Q, long long sQ, const void* X,
                 long long sX, int out_dtype, void* Y, long long sY, float alpha, hipStream_t s,
                 bool rev = false) {
  GemmArgs g;
  g.reverse = rev;
  g.op = OP_GEMM; g.dtype = in_dtype; g.out_dtype = out_dtype; g.batch = batch;
  g.M = k; g.N = m; g.K = k;
  g.A = Q; g.lda = k; g.sA = sQ;
  g.B = X; g.ldb = m; g.sB = sX;
  g.E = nullptr; g.lde = 0; g.sE = 0;
  g.C = Y; g.ldc = m; g.sC = sY;
  g.alpha = alpha; g.beta = 0.f; g.gamma = 0.f;
  return launch_gemm(g, s);
}

// The last product O = Q X of a call: one launch, or with fu, one launch per
// segment, fused with the update of W where the segment asks for it and the
// large-tile kernel runs the product.
static int final_qx(int batch, int k, int m, int dt, const void* Q, long long sQ, const void* X, long long sX,
                    void* O, long long sO, hipStream_t s, bool rev, FusedUpdate* fu) {
  if (!fu) return qx_op(batch, k, m, dt, Q, sQ, X, sX, dt, O, sO, 1.f, s, rev);
  const size_t es = dtype_size(dt);
  int st = DION3_OK;
  for (int i = 0; i < fu->nseg && st == DION3_OK; ++i) {
    FusedSegment& g = fu->seg[i];
    g.fused = false;
    if (g.nb < 1 || g.b0 < 0 || g.b0 + g.nb > batch) return DION3_ERR_INVALID_ARG;
    const char* q = (const char*)Q + (size_t)g.b0 * sQ * es;
    const char* x = (const char*)X + (size_t)g.b0 * sX * es;
    char* o = (char*)O + (size_t)g.b0 * sO * es;
    GemmArgs a;
    a.op = OP_GEMM; a.dtype = dt; a.out_dtype = dt; a.batch = g.nb;
    a.M = k; a.N = m; a.K = k;
    a.A = q; a.lda = k; a.sA = sQ;
    a.B = x; a.ldb = m; a.sB = sX;
    a.E = nullptr; a.lde = 0; a.sE = 0;
    a.C = o; a.ldc = m; a.sC = sO;
    a.alpha = 1.f; a.beta = 0.f; a.gamma = 0.f;
    a.reverse = rev;
    GemmArgs f = a;
    f.W = g.W; f.sW = g.sW; f.wlines = g.wlines; f.idx = g.idx;
    f.eta = fu->eta; f.u = fu->u; f.decay = fu->decay;
    if (g.fuse && gemm_fused_update_ok(f)) {
      st = launch_gemm(f, s);
      g.fused = st == DION3_OK;
    } else {
      st = launch_gemm(a, s);
    }
  }
  return st;
}

static bool ns_dtype_ok(int dt) { return dt == DION3_F16 || dt == DION3_F32 || dt == DION3_BF16; }

}  // namespace dion3

using namespace dion3;

extern "C" int dion3_syrk(int batch, int n, int kdim, int dtype, const void* A, long long strideA,
                          void* C, long long strideC, float alpha, float beta, void* stream) {
  if (batch < 1 || n < 1 || kdim < 1 || !A || !C || !ns_dtype_ok(dtype)) return DION3_ERR_INVALID_ARG;
  if (A == C) return DION3_ERR_INVALID_ARG;
  if (batch > 1 && (strideA < (long long)n * kdim || strideC < (long long)n * n)) return DION3_ERR_INVALID_ARG;
  return sym_op(OP_SYRK, batch, n, kdim, dtype, A, strideA, A, strideA, beta != 0.f ? C : nullptr,
                strideC, C, strideC, alpha, beta, 0.f, (hipStream_t)stream);
}

extern "C" int dion3_sym_sq_add(int batch, int n, int dtype, const void* A, long long strideA,
                                const void* B, long long strideB, void* C, long long strideC,
                                float alpha, float beta, float gamma, void* stream) {
  if (batch < 1 || n < 1 || !A || !B || !C || !ns_dtype_ok(dtype)) return DION3_ERR_INVALID_ARG;
  if (C == A || C == B) return DION3_ERR_INVALID_ARG;
  const long long nn = (long long)n * n;
  if (batch > 1 && (strideA < nn || strideB < nn || strideC < nn)) return DION3_ERR_INVALID_ARG;
  return sym_op(OP_SQ_ADD, batch, n, n, dtype, A, strideA, A, strideA, B, strideB, C, strideC, alpha,
                beta, gamma, (hipStream_t)stream);
}

extern "C" int dion3_sym_mul(int batch, int n, int dtype, const void* A, long long strideA,
                             const void* B, long long strideB, void* C, long long strideC,
                             float alpha, void* stream) {
  if (batch < 1 || n < 1 || !A || !B || !C || !ns_dtype_ok(dtype)) return DION3_ERR_INVALID_ARG;
  if (C == A || C == B) return DION3_ERR_INVALID_ARG;
  const long long nn = (long long)n * n;
  if (batch > 1 && (strideA < nn || strideB < nn || strideC < nn)) return DION3_ERR_INVALID_ARG;
  return sym_op(OP_SYM_MUL, batch, n, n, dtype, A, strideA, B, strideB, nullptr, 0, C, strideC, alpha,
                0.f, 0.f, (hipStream_t)stream);
}

extern "C" int dion3_gemm(int batch, int k, int m, int in_dtype, const void* Q, long long strideQ,
                          const void* X, long long strideX, int out_dtype, void* Y, long long strideY,
                          float alpha, void* stream) {
  if (batch < 1 || k < 1 || m < 1 || !Q || !X || !Y || !ns_dtype_ok(in_dtype)) return DION3_ERR_INVALID_ARG;
  if (Y == Q || Y == X) return DION3_ERR_INVALID_ARG;
  if (!(out_dtype == in_dtype || (in_dtype == DION3_F16 && out_dtype == DION3_F32)))
    return DION3_ERR_INVALID_ARG;
  if (batch > 1 && (strideQ < (long long)k * k || strideX < (long long)k * m || strideY < (long long)k * m))
    return DION3_ERR_INVALID_ARG;
  return qx_op(batch, k, m, in_dtype, Q, strideQ, X, strideX, out_dtype, Y, strideY, alpha,
               (hipStream_t)stream);
}

extern "C" size_t dion3_gram_ns_gathered_workspace_bytes(int batch, int k, int m, int ns_dtype) {
  if (batch < 1 || k < 1 || m < 1 || !ns_dtype_ok(ns_dtype)) return 0;
  const size_t es = dtype_size(ns_dtype);
  return align256((size_t)batch * k * m * es) + 4 * align256((size_t)batch * k * k * es);
}

namespace dion3 {
int gram_ns_gathered_fused(int batch, int k, int m, const dion3_ns_params* p, const void* X0, void* O, void* ws,
                           size_t ws_bytes, void* stream, FusedUpdate* fu) {
  if (batch < 1 || k < 1 || m < 1 || k > m || !p || !X0 || !O || X0 == O) return DION3_ERR_INVALID_ARG;
  if (p->T < 1 || !p->coeffs || !ns_dtype_ok(p->ns_dtype)) return DION3_ERR_INVALID_ARG;
  for (int i = 0; i < 3 * p->T; ++i)
    if (!(p->coeffs[i] == p->coeffs[i])) return DION3_ERR_INVALID_ARG;
  const size_t need = dion3_gram_ns_gathered_workspace_bytes(batch, k, m, p->ns_dtype);
  if (!ws || ws_bytes < need) return DION3_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int dt = p->ns_dtype;
  const size_t es = dtype_size(dt);
  const long long skm = (long long)k * m, skk = (long long)k * k;
  char* w = (char*)ws;
  void* X2 = w;
  void* sq[4];
  char* base = w + align256((size_t)batch * skm * es);
  for (int i = 0; i < 4; ++i) sq[i] = base + i * align256((size_t)batch * skk * es);

  // iteration boundaries of the passes
  int bounds[66];
  int nb = 0;
  bounds[nb++] = 0;
  for (int t = 1; t < p->T && t < 64; ++t)
    if ((p->restart_mask >> t) & 1u) bounds[nb++] = t;
  bounds[nb++] = p->T;
  const int npass = nb - 1;

  bool used[4] = {false, false, false, false};
  auto take = [&]() -> int {
    for (int i = 0; i < 4; ++i)
      if (!used[i]) { used[i] = true; return i; }
    return -1;
  };
  auto give = [&](int i) { if (i >= 0) used[i] = false; };

  // Consecutive products visit the batch in opposite orders, so each starts on
  // the matrices the previous one finished last, whose operands the
  // last-level cache may still hold (the first starts at the end the gather
  // wrote last).
  bool rev = true;
  auto order = [&]() { const bool r = rev; rev = !rev; return r; };

  const void* cur = X0;
  int st = DION3_OK;
  for (int ps = 0; ps < npass && st == DION3_OK; ++ps) {
    const int t0 = bounds[ps], t1 = bounds[ps + 1];
    void* out = ((npass - 1 - ps) % 2 == 0) ? O : X2;
    const int R = take();
    st = sym_op(OP_SYRK, batch, k, m, dt, cur, skm, cur, skm, nullptr, 0, sq[R], skk, 1.f, 0.f, 0.f, s,
                order());
    int Q = -1;
    for (int t = t0; t < t1 && st == DION3_OK; ++t) {
      const float a = (float)p->coeffs[3 * t + 0];
      const float b = (float)p->coeffs[3 * t + 1];
      const float c = (float)p->coeffs[3 * t + 2];
      const int Z = take();
      st = sym_op(OP_SQ_ADD, batch, k, k, dt, sq[R], skk, sq[R], skk, sq[R], skk, sq[Z], skk, c, b, a, s,
                  order());
      if (st) break;
      if (Q < 0) {
        Q = Z;
      } else {
        const int Qn = take();
        st = sym_op(OP_SYM_MUL, batch, k, k, dt, sq[Q], skk, sq[Z], skk, nullptr, 0, sq[Qn], skk, 1.f, 0.f,
                    0.f, s, order());
        give(Q);
        Q = Qn;
        if (st) break;
      }
      if (t < t1 - 1) {
        const int P = take();
        st = sym_op(OP_SYM_MUL, batch, k, k, dt, sq[Z], skk, sq[R], skk, nullptr, 0, sq[P], skk, 1.f, 0.f,
                    0.f, s, order());
        if (!st)
          st = sym_op(OP_SYM_MUL, batch, k, k, dt, sq[P], skk, sq[Z], skk, nullptr, 0, sq[R], skk, 1.f, 0.f,
                      0.f, s, order());
        give(P);
      }
      if (Z != Q) give(Z);
    }
    if (st) break;
    if (ps == npass - 1)
      st = final_qx(batch, k, m, dt, sq[Q], skk, cur, skm, out, skm, s, order(), fu);
    else
      st = qx_op(batch, k, m, dt, sq[Q], skk, cur, skm, dt, out, skm, 1.f, s, order());
    give(Q);
    give(R);
    cur = out;
  }
  return st;
}
}  // namespace dion3

extern "C" int dion3_gram_ns_gathered(int batch, int k, int m, const dion3_ns_params* p, const void* X0,
                                      void* O, void* ws, size_t ws_bytes, void* stream) {
  return gram_ns_gathered_fused(batch, k, m, p, X0, O, ws, ws_bytes, stream, nullptr);
}

// Gram Newton-Schulz of a group's selected submatrices, from M and the
// selection ("Dion3: Full-Stack Orthogonal Updates", Section 2 for the
// Frobenius normalisation of the input, Section 4 for the iteration).  The
// workspace holds the per-line and per-matrix sums of squares, X0 and the
// scratch of the gathered form.
static size_t gram_group_parts(const dion3_group* g, int k, const dion3_ns_params* p, int* n, int* m,
                               int* axis, size_t part[4]) {
  if (!p || !canonical_dims(g, n, m, axis) || k < 1 || k > *n || k > *m || !ns_dtype_ok(p->ns_dtype)) return 0;
  const size_t es = dtype_size(p->ns_dtype);
  part[0] = align256((size_t)g->batch * k * sizeof(double));    // per-line sums of squares
  part[1] = align256((size_t)g->batch * sizeof(double));        // ||M[S,:]||_F^2 per matrix
  part[2] = align256((size_t)g->batch * k * *m * es);           // X0
  part[3] = dion3_gram_ns_gathered_workspace_bytes(g->batch, k, *m, p->ns_dtype);
  return part[3] ? part[0] + part[1] + part[2] + part[3] : 0;
}

extern "C" size_t dion3_gram_ns_workspace_bytes(const dion3_group* g, int k, const dion3_ns_params* p) {
  int n, m, axis;
  size_t part[4];
  return gram_group_parts(g, k, p, &n, &m, &axis, part);
}

extern "C" size_t dion3_workspace_bytes(const dion3_group* g, int k, const dion3_ns_params* p) {
  const size_t a = dion3_rowsel_workspace_bytes(g);
  const size_t b = dion3_gram_ns_workspace_bytes(g, k, p);
  if (!a || !b) return 0;
  return a > b ? a : b;
}

extern "C" int dion3_gram_ns(const dion3_group* g, const void* M, const int32_t* idx, int k,
                             const dion3_ns_params* p, void* O, void* ws, size_t ws_bytes, void* stream) {
  int n, m, axis;
  size_t part[4];
  const size_t need = gram_group_parts(g, k, p, &n, &m, &axis, part);
  if (!need || !M || !idx || !O) return DION3_ERR_INVALID_ARG;
  // the gather writes X0 in fp16 or fp32 from bf16 or fp32 storage
  if (g->dtype != DION3_F32 && g->dtype != DION3_BF16) return DION3_ERR_INVALID_ARG;
  if (p->ns_dtype != DION3_F16 && p->ns_dtype != DION3_F32) return DION3_ERR_INVALID_ARG;
  if (p->T < 1 || !p->coeffs || !(p->eps >= 0.f)) return DION3_ERR_INVALID_ARG;
  for (int i = 0; i < 3 * p->T; ++i)
    if (!(p->coeffs[i] == p->coeffs[i])) return DION3_ERR_INVALID_ARG;
  if (!ws || ws_bytes < need) return DION3_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  double* lines = (double*)w;
  double* sqn = (double*)(w + part[0]);
  void* X0 = w + part[0] + part[1];
  void* scratch = w + part[0] + part[1] + part[2];
  int st = selected_sqnorm(g, axis, M, idx, k, lines, sqn, s);
  if (!st) st = dion3_gather_rows(g, M, idx, k, sqn, p->eps, p->ns_dtype, X0, stream);
  if (!st) st = dion3_gram_ns_gathered(g->batch, k, m, p, X0, O, scratch, part[3], stream);
  return st;
}

// Standard Newton-Schulz on the same symmetric kernels ("Dion3: Full-Stack
// Orthogonal Updates", Section 2 for the iteration; Section 4 and Appendix C.3
// for the fall-back when the aspect ratio is 1).  Per iteration on X:
//   A = X X^T                  (symmetric kernel, lower triangle + mirror)
//   Z = a I + b A + c A^2      (A^2 + B kernel, the identity in its epilogue)
//   X <- Z X                   (rectangular kernel)
// which is X <- a X + (b A + c A^2) X with the a X term carried by Z.
// Buffers: X0 read only; outputs alternate between a k x m workspace slice
// and O so that the last iteration writes O; two k x k slices hold A and Z.
extern "C" size_t dion3_standard_ns_workspace_bytes(int batch, int k, int m, int ns_dtype) {
  if (batch < 1 || k < 1 || m < 1 || !ns_dtype_ok(ns_dtype)) return 0;
  const size_t es = dtype_size(ns_dtype);
  return align256((size_t)batch * k * m * es) + 2 * align256((size_t)batch * k * k * es);
}

namespace dion3 {
int standard_ns_fused(int batch, int k, int m, const dion3_ns_params* p, const void* X0, void* O, void* ws,
                      size_t ws_bytes, void* stream, FusedUpdate* fu) {
  if (batch < 1 || k < 1 || m < 1 || k > m || !p || !X0 || !O || X0 == O) return DION3_ERR_INVALID_ARG;
  if (p->T < 1 || !p->coeffs || !ns_dtype_ok(p->ns_dtype)) return DION3_ERR_INVALID_ARG;
  for (int i = 0; i < 3 * p->T; ++i)
    if (!(p->coeffs[i] == p->coeffs[i])) return DION3_ERR_INVALID_ARG;
  const size_t need = dion3_standard_ns_workspace_bytes(batch, k, m, p->ns_dtype);
  if (!ws || ws_bytes < need) return DION3_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int dt = p->ns_dtype;
  const size_t es = dtype_size(dt);
  const long long skm = (long long)k * m, skk = (long long)k * k;
  char* w = (char*)ws;
  void* Xw = w;
  void* A = w + align256((size_t)batch * skm * es);
  void* Z = (char*)A + align256((size_t)batch * skk * es);
  bool rev = true;     // alternate batch orders, as in the Gram form
  auto order = [&]() { const bool r = rev; rev = !rev; return r; };
  const void* cur = X0;
  int st = DION3_OK;
  for (int t = 0; t < p->T && st == DION3_OK; ++t) {
    const float a = (float)p->coeffs[3 * t + 0];
    const float b = (float)p->coeffs[3 * t + 1];
    const float c = (float)p->coeffs[3 * t + 2];
    void* out = ((p->T - 1 - t) % 2 == 0) ? O : Xw;
    st = sym_op(OP_SYRK, batch, k, m, dt, cur, skm, cur, skm, nullptr, 0, A, skk, 1.f, 0.f, 0.f, s, order());
    if (!st) st = sym_op(OP_SQ_ADD, batch, k, k, dt, A, skk, A, skk, A, skk, Z, skk, c, b, a, s, order());
    if (!st)
      st = t == p->T - 1 ? final_qx(batch, k, m, dt, Z, skk, cur, skm, out, skm, s, order(), fu)
                         : qx_op(batch, k, m, dt, Z, skk, cur, skm, dt, out, skm, 1.f, s, order());
    cur = out;
  }
  return st;
}
}  // namespace dion3

extern "C" int dion3_standard_ns(int batch, int k, int m, const dion3_ns_params* p, const void* X0,
                                 void* O, void* ws, size_t ws_bytes, void* stream) {
  return standard_ns_fused(batch, k, m, p, X0, O, ws, ws_bytes, stream, nullptr);
}
