// Whole-step driver: momentum + selection, gather, batched Gram Newton-Schulz
// per canonical shape, and the fused update, all enqueued on one stream.
//
// Method: "Dion3: Full-Stack Orthogonal Updates", Section 6 (update rule) and
// Section 7 (megabatching: every matrix of one shape is processed as one
// batch).  On one GPU the batching is across launches: matrices whose selected
// submatrices have the same (k, m) share one Newton-Schulz batch, so an
// up-projection group (row selection) and a down-projection group (column
// selection, stored transposed) run their Newton-Schulz together.
#include <vector>

#include "common.h"

namespace dion3 {
static inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Plan {
  std::vector<int> n, m, axis;
  std::vector<std::vector<int>> classes;   // groups sharing (k, m), in order of first appearance
  size_t rowsel = 0, xbuf = 0, gram = 0;
};

static bool make_plan(int ng, const dion3_group* g, const int* k, const dion3_ns_params* p, Plan& P) {
  if (ng < 1 || !g || !k || !p) return false;
  P.n.resize(ng); P.m.resize(ng); P.axis.resize(ng);
  const size_t es = dtype_size(p->ns_dtype);
  if (!es) return false;
  for (int i = 0; i < ng; ++i) {
    if (!canonical_dims(&g[i], &P.n[i], &P.m[i], &P.axis[i])) return false;
    if (k[i] < 1 || k[i] > P.n[i]) return false;
    P.rowsel = std::max(P.rowsel, al256(dion3_rowsel_workspace_bytes(&g[i])) + al256(g[i].batch * sizeof(double)));
    bool placed = false;
    for (auto& c : P.classes)
      if (k[c[0]] == k[i] && P.m[c[0]] == P.m[i]) { c.push_back(i); placed = true; break; }
    if (!placed) P.classes.push_back({i});
  }
  for (auto& c : P.classes) {
    int nb = 0;
    for (int i : c) nb += g[i].batch;
    const int kk = k[c[0]], mm = P.m[c[0]];
    P.xbuf = std::max(P.xbuf, al256((size_t)nb * kk * mm * es));
    P.gram = std::max(P.gram, dion3_gram_ns_workspace_bytes(nb, kk, mm, p->ns_dtype));
  }
  return true;
}
}  // namespace dion3

using namespace dion3;

extern "C" size_t dion3_step_workspace_bytes(int n_groups, const dion3_group* groups, const int* k,
                                             const dion3_ns_params* p) {
  Plan P;
  if (!make_plan(n_groups, groups, k, p, P)) return 0;
  return P.rowsel + 2 * P.xbuf + P.gram;
}

static int run_step(int n_groups, const dion3_group* groups, void* const* W, void* const* M,
                    const void* const* G, const int* k, int32_t* const* idx,
                    const dion3_ns_params* p, float eta, float wd, float mu, void* ws,
                    size_t ws_bytes, void* stream, bool deferred, bool has_prev) {
  Plan P;
  if (!W || !M || !G || !idx || !make_plan(n_groups, groups, k, p, P)) return DION3_ERR_INVALID_ARG;
  for (int i = 0; i < n_groups; ++i)
    if (!W[i] || !M[i] || !G[i] || !idx[i]) return DION3_ERR_INVALID_ARG;
  const size_t need = P.rowsel + 2 * P.xbuf + P.gram;
  if (!ws || ws_bytes < need) return DION3_ERR_WORKSPACE;
  char* base = (char*)ws;
  char* rs_ws = base;
  char* X0 = base + P.rowsel;
  char* O = X0 + P.xbuf;
  char* gws = O + P.xbuf;
  const size_t es = dtype_size(p->ns_dtype);
  int st = DION3_OK;
  for (auto& c : P.classes) {
    const int kk = k[c[0]], mm = P.m[c[0]];
    const size_t slice = (size_t)kk * mm * es;
    int nb = 0;
    for (int i : c) {
      const dion3_group& gi = groups[i];
      const size_t rsz = al256(dion3_rowsel_workspace_bytes(&gi));
      double* sqn = (double*)(rs_ws + rsz);
      // deferred error feedback: idx[i] holds the previous selection on entry;
      // its decay is applied in this pass, then idx[i] is overwritten
      st = dion3_momentum_rowsel_ef(&gi, M[i], G[i], kk, idx[i], nullptr, sqn,
                                    deferred && has_prev ? idx[i] : nullptr, kk, mu, rs_ws, rsz, stream);
      if (st) return st;
      st = dion3_gather_rows(&gi, M[i], idx[i], kk, sqn, p->eps, p->ns_dtype, X0 + nb * slice, stream);
      if (st) return st;
      nb += gi.batch;
    }
    st = dion3_gram_ns(nb, kk, mm, p, X0, O, gws, P.gram, stream);
    if (st) return st;
    nb = 0;
    for (int i : c) {
      const dion3_group& gi = groups[i];
      st = dion3_apply_rows(&gi, W[i], deferred ? nullptr : M[i], idx[i], kk, O + nb * slice, p->ns_dtype,
                            (long long)kk * mm, eta, wd, mu, stream);
      if (st) return st;
      nb += gi.batch;
    }
  }
  return st;
}

extern "C" int dion3_step(int n_groups, const dion3_group* groups, void* const* W, void* const* M,
                          const void* const* G, const int* k, int32_t* const* idx,
                          const dion3_ns_params* p, float eta, float wd, float mu, void* ws,
                          size_t ws_bytes, void* stream) {
  return run_step(n_groups, groups, W, M, G, k, idx, p, eta, wd, mu, ws, ws_bytes, stream, false, false);
}

extern "C" int dion3_step_deferred(int n_groups, const dion3_group* groups, void* const* W,
                                   void* const* M, const void* const* G, const int* k,
                                   int32_t* const* idx, int has_prev, const dion3_ns_params* p,
                                   float eta, float wd, float mu, void* ws, size_t ws_bytes,
                                   void* stream) {
  return run_step(n_groups, groups, W, M, G, k, idx, p, eta, wd, mu, ws, ws_bytes, stream, true,
                  has_prev != 0);
}
