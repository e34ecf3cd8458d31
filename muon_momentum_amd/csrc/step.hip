// Whole-step driver: momentum + selection, gather, batched Gram Newton-Schulz
// per canonical shape, and the fused update.
//
// Method: "Dion3: Full-Stack Orthogonal Updates", Section 6 (update rule) and
// Section 7 (megabatching: every matrix of one shape is processed as one
// batch).  On one GPU the batching is across launches: matrices whose selected
// submatrices have the same (k, m) share one Newton-Schulz batch, so an
// up-projection group (row selection) and a down-projection group (column
// selection, stored transposed) run their Newton-Schulz together.
//
// Two streams.  The HBM-bound passes (momentum + selection of every group,
// then the update of each class) run on the caller's stream; the gathers and
// the matrix-core-bound Newton-Schulz chain of each class run on a side
// stream owned by the library, so the momentum pass of later classes and the
// update of earlier ones overlap the products of the current class.  Events
// order the two: class c's gather waits for its groups' selection, class c's
// update waits for its Newton-Schulz, and the caller's stream ends the call
// having waited for all side-stream work.  Every kernel computes exactly what
// it computes on one stream, so the results do not depend on the overlap.
#include <mutex>
#include <vector>

#include "common.h"

namespace dion3 {
static inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Plan {
  std::vector<int> n, m, axis;
  std::vector<std::vector<int>> classes;   // groups sharing (k, m), in order of first appearance
  std::vector<size_t> sqn_off;             // per group: offset of its [batch] fp64 slot
  size_t rowsel = 0, sqn = 0, xbuf = 0, gram = 0;
  size_t bytes() const { return rowsel + sqn + (classes.size() > 1 ? 3 : 2) * xbuf + gram; }
};

static bool make_plan(int ng, const dion3_group* g, const int* k, const dion3_ns_params* p, Plan& P) {
  if (ng < 1 || !g || !k || !p) return false;
  P.n.resize(ng); P.m.resize(ng); P.axis.resize(ng); P.sqn_off.resize(ng);
  const size_t es = dtype_size(p->ns_dtype);
  if (!es) return false;
  for (int i = 0; i < ng; ++i) {
    if (!canonical_dims(&g[i], &P.n[i], &P.m[i], &P.axis[i])) return false;
    if (k[i] < 1 || k[i] > P.n[i]) return false;
    P.rowsel = std::max(P.rowsel, al256(dion3_rowsel_workspace_bytes(&g[i])));
    P.sqn_off[i] = P.sqn;
    P.sqn += al256(g[i].batch * sizeof(double));
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

// The side stream (default priority, not synchronising with the null stream)
// and an event pool, created on a device's first step and kept until the
// process ends.  Enqueueing a step holds the mutex, so concurrent callers do
// not interleave their use of the events.
struct SideCtx {
  hipStream_t side = nullptr;
  std::vector<hipEvent_t> ev;
};
constexpr int kMaxDevices = 64;
static std::mutex g_side_mu;
static SideCtx g_side[kMaxDevices];

static int side_ctx(size_t nev, SideCtx** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DION3_ERR_HIP;
  SideCtx& c = g_side[dev];
  if (!c.side && hipStreamCreateWithFlags(&c.side, hipStreamNonBlocking) != hipSuccess) {
    c.side = nullptr;
    return DION3_ERR_HIP;
  }
  while (c.ev.size() < nev) {
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return DION3_ERR_HIP;
    c.ev.push_back(e);
  }
  *out = &c;
  return DION3_OK;
}
}  // namespace dion3

using namespace dion3;

extern "C" size_t dion3_step_workspace_bytes(int n_groups, const dion3_group* groups, const int* k,
                                             const dion3_ns_params* p) {
  Plan P;
  if (!make_plan(n_groups, groups, k, p, P)) return 0;
  return P.bytes();
}

static int run_step(int n_groups, const dion3_group* groups, void* const* W, void* const* M,
                    const void* const* G, const int* k, int32_t* const* idx,
                    const dion3_ns_params* p, float eta, float wd, float mu, void* ws,
                    size_t ws_bytes, void* stream, bool deferred, bool has_prev) {
  Plan P;
  if (!W || !M || !G || !idx || !make_plan(n_groups, groups, k, p, P)) return DION3_ERR_INVALID_ARG;
  for (int i = 0; i < n_groups; ++i)
    if (!W[i] || !M[i] || !G[i] || !idx[i]) return DION3_ERR_INVALID_ARG;
  if (!ws || ws_bytes < P.bytes()) return DION3_ERR_WORKSPACE;
  const int nc = (int)P.classes.size();
  // workspace: top-k partials | per-group selected sums of squares | X0 |
  // outputs of alternate classes (two while a class's update may still read
  // the previous output) | Newton-Schulz scratch
  char* base = (char*)ws;
  char* rs_ws = base;
  char* sqn_base = rs_ws + P.rowsel;
  char* X0 = sqn_base + P.sqn;
  char* Obuf[2] = {X0 + P.xbuf, X0 + (nc > 1 ? 2 : 1) * P.xbuf};
  char* gws = X0 + (nc > 1 ? 3 : 2) * P.xbuf;
  const size_t es = dtype_size(p->ns_dtype);
  hipStream_t s = (hipStream_t)stream;

  std::lock_guard<std::mutex> lock(g_side_mu);
  SideCtx* ctx = nullptr;
  int st = side_ctx(3 * (size_t)nc + 1, &ctx);
  if (st) return st;
  hipStream_t side = ctx->side;
  hipEvent_t* ev_sel = ctx->ev.data();          // class c selected (caller's stream)
  hipEvent_t* ev_ns = ev_sel + nc;              // class c orthogonalised (side stream)
  hipEvent_t* ev_upd = ev_ns + nc;              // class c updated (caller's stream)
  hipEvent_t ev_end = ev_upd[nc];               // side stream drained
  auto hip_ok = [](hipError_t e) { return e == hipSuccess ? DION3_OK : DION3_ERR_HIP; };

  // caller's stream: momentum + selection of every group, class by class
  for (int c = 0; c < nc && !st; ++c) {
    for (int i : P.classes[c]) {
      const dion3_group& gi = groups[i];
      // deferred error feedback: idx[i] holds the previous selection on entry;
      // its decay is applied in this pass, then idx[i] is overwritten
      st = dion3_momentum_rowsel_ef(&gi, M[i], G[i], k[i], idx[i], nullptr,
                                    (double*)(sqn_base + P.sqn_off[i]),
                                    deferred && has_prev ? idx[i] : nullptr, k[i], mu, rs_ws,
                                    P.rowsel, s);
      if (st) break;
    }
    if (!st) st = hip_ok(hipEventRecord(ev_sel[c], s));
  }
  // per class: gather + Newton-Schulz on the side stream, update on the caller's
  bool forked = false;
  for (int c = 0; c < nc && !st; ++c) {
    const auto& cls = P.classes[c];
    const int kk = k[cls[0]], mm = P.m[cls[0]];
    const size_t slice = (size_t)kk * mm * es;
    char* O = Obuf[c & 1];
    st = hip_ok(hipStreamWaitEvent(side, ev_sel[c], 0));
    forked = forked || !st;
    // O is rewritten two classes later: wait until that class's update read it
    if (!st && c >= 2) st = hip_ok(hipStreamWaitEvent(side, ev_upd[c - 2], 0));
    int nb = 0;
    for (int i : cls) {
      if (st) break;
      const dion3_group& gi = groups[i];
      st = dion3_gather_rows(&gi, M[i], idx[i], kk, (const double*)(sqn_base + P.sqn_off[i]), p->eps,
                             p->ns_dtype, X0 + nb * slice, side);
      nb += gi.batch;
    }
    if (!st) st = dion3_gram_ns(nb, kk, mm, p, X0, O, gws, P.gram, side);
    if (!st) st = hip_ok(hipEventRecord(ev_ns[c], side));
    if (!st) st = hip_ok(hipStreamWaitEvent(s, ev_ns[c], 0));
    nb = 0;
    for (int i : cls) {
      if (st) break;
      const dion3_group& gi = groups[i];
      st = dion3_apply_rows(&gi, W[i], deferred ? nullptr : M[i], idx[i], kk, O + nb * slice, p->ns_dtype,
                            (long long)kk * mm, eta, wd, mu, s);
      nb += gi.batch;
    }
    if (!st) st = hip_ok(hipEventRecord(ev_upd[c], s));
  }
  // join: the caller's stream waits for everything enqueued on the side stream
  // (also after an error, so that no side-stream work outlives the call's order)
  if (forked) {
    const int j = hip_ok(hipEventRecord(ev_end, side));
    const int w = j ? j : hip_ok(hipStreamWaitEvent(s, ev_end, 0));
    if (!st) st = w;
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
