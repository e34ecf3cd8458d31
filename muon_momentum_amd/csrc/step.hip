// Whole-step driver: momentum + selection, gather, batched Gram Newton-Schulz
// per canonical shape, and the fused update.
//
// Method: "Dion3: Full-Stack Orthogonal Updates", Section 6 (update rule),
// Section 7 (megabatching: every matrix of one shape is processed as one
// batch), Section 2 for the NorMuon flavour, and Section 4 (a class whose selected submatrices are square uses
// standard Newton-Schulz on the symmetric kernels, Gram Newton-Schulz
// otherwise).  On one GPU the batching is across launches: matrices whose selected
// submatrices have the same (k, m) share one Newton-Schulz batch, so an
// up-projection group (row selection) and a down-projection group (column
// selection, stored transposed) run their Newton-Schulz together.
//
// Three streams.  The matrix-core-bound Newton-Schulz chain of each class
// runs on a side stream owned by the library.  The first class's momentum +
// selection pass and its gather have nothing to overlap and run on the
// caller's stream over the whole chip, and so does the last class's update;
// the momentum passes and gathers of the other classes and the updates of all
// but the last run on a second library stream, in the order momentum and
// gather of class c + 1, then update of class c, so that these HBM-bound
// passes overlap the products of class c.  When those momentum passes are
// large that stream is restricted to half of the compute units (spread evenly
// over the XCDs), so that they do not take every unit from the products;
// small ones run on every unit.  Events order the streams: class c's Newton-Schulz waits for its
// gather, class c's update for its Newton-Schulz, a gather for the end of the
// Newton-Schulz that last read its buffer, and the caller's stream ends the
// call having waited for all library-stream work.  Every kernel computes
// exactly what it computes on one stream, so the results do not depend on
// the overlap.
#include <algorithm>
#include <mutex>
#include <vector>

#include "common.h"

namespace dion3 {
static inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Plan {
  std::vector<int> n, m, axis;
  std::vector<std::vector<int>> classes;   // groups sharing (k, m), by increasing momentum traffic
  std::vector<size_t> sqn_off;             // per group: offset of its [batch] fp64 slot
  std::vector<size_t> rs_off;              // per group: offset of its [batch][k] fp32 row factors
  size_t rowsel = 0, sqn = 0, rs = 0, xbuf = 0, gram = 0;
  size_t bytes() const { return rowsel + sqn + rs + (classes.size() > 1 ? 4 : 2) * xbuf + gram; }
};

static bool make_plan(int ng, const dion3_group* g, const int* k, const dion3_ns_params* p, Plan& P) {
  if (ng < 1 || !g || !k || !p) return false;
  P.n.resize(ng); P.m.resize(ng); P.axis.resize(ng); P.sqn_off.resize(ng); P.rs_off.resize(ng);
  // the gather and the update pass take fp16 or fp32 Newton-Schulz buffers
  // and bf16 or fp32 storage: any other pair is refused here, before any launch
  if (p->ns_dtype != DION3_F16 && p->ns_dtype != DION3_F32) return false;
  const size_t es = dtype_size(p->ns_dtype);
  for (int i = 0; i < ng; ++i) {
    if (g[i].dtype != DION3_BF16 && g[i].dtype != DION3_F32) return false;
    if (!canonical_dims(&g[i], &P.n[i], &P.m[i], &P.axis[i])) return false;
    if (k[i] < 1 || k[i] > P.n[i]) return false;
    P.rowsel = std::max(P.rowsel, al256(dion3_rowsel_workspace_bytes(&g[i])));
    P.sqn_off[i] = P.sqn;
    P.sqn += al256(g[i].batch * sizeof(double));
    P.rs_off[i] = P.rs;
    P.rs += al256((size_t)g[i].batch * k[i] * sizeof(float));
    bool placed = false;
    for (auto& c : P.classes)
      if (k[c[0]] == k[i] && P.m[c[0]] == P.m[i]) { c.push_back(i); placed = true; break; }
    if (!placed) P.classes.push_back({i});
  }
  // the first class's momentum pass has nothing beside it and the last
  // class's products have no momentum pass beside them: the class with the
  // least momentum traffic goes first (7B set: 26.0 against 27.0 ms per step
  // with the larger class first), whatever the order of the groups
  auto traffic = [&](const std::vector<int>& c) {
    double t = 0.0;
    for (int i : c) t += (double)dtype_size(g[i].dtype) * g[i].rows * g[i].cols * g[i].batch;
    return t;
  };
  std::stable_sort(P.classes.begin(), P.classes.end(),
                   [&](const std::vector<int>& a, const std::vector<int>& b) { return traffic(a) < traffic(b); });
  for (auto& c : P.classes) {
    int nb = 0;
    for (int i : c) nb += g[i].batch;
    const int kk = k[c[0]], mm = P.m[c[0]];
    P.xbuf = std::max(P.xbuf, al256((size_t)nb * kk * mm * es));
    P.gram = std::max(P.gram, mm == kk ? dion3_standard_ns_workspace_bytes(nb, kk, mm, p->ns_dtype)
                                       : dion3_gram_ns_gathered_workspace_bytes(nb, kk, mm, p->ns_dtype));
  }
  return true;
}

// The library streams (default priority) and an event pool, each created
// when a step on the device first needs it and kept until dion3_release or
// the end of the process.  Enqueueing a step
// holds the mutex, so concurrent callers do not interleave their use of the
// events.  The compute-unit-masked stream is a blocking stream (its creation
// call takes no flags, so it synchronises with the legacy null stream).
struct SideCtx {
  hipStream_t side = nullptr;   // gathers + Newton-Schulz, every compute unit (non-blocking)
  hipStream_t mem = nullptr;    // overlapped HBM-bound passes, half the compute units (blocking)
  hipStream_t mem_all = nullptr;  // the same passes on every unit, for small steps (non-blocking)
  std::vector<hipEvent_t> ev;
  unsigned gen = 0;             // set when the streams are created (step graphs check it)
};
constexpr int kMaxDevices = 64;
constexpr double kMaskedOverlapBytes = 8e9;   // see run_step
static std::mutex g_side_mu;
static SideCtx g_side[kMaxDevices];
static unsigned g_side_gen = 0;

std::mutex& side_mutex() { return g_side_mu; }

// Generation of the current device's library streams (0: none); the caller
// holds side_mutex().
unsigned side_generation() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  return g_side[dev].side ? g_side[dev].gen : 0;
}

// Compute-unit mask of the overlapped stream: unit i is used when
// (i mod 8 + i div 8) mod 8 < 4, which takes half of the units of every XCD
// whether the units are numbered XCD by XCD or interleaved across XCDs.
static int make_mem_stream(int dev, hipStream_t* out) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 16)
    return hipStreamCreateWithFlags(out, hipStreamNonBlocking) == hipSuccess ? DION3_OK : DION3_ERR_HIP;
  std::vector<uint32_t> mask((cus + 31) / 32, 0u);
  for (int i = 0; i < cus; ++i)
    if ((i % 8 + i / 8) % 8 < 4) mask[i / 32] |= 1u << (i % 32);
  return hipExtStreamCreateWithCUMask(out, (uint32_t)mask.size(), mask.data()) == hipSuccess ? DION3_OK
                                                                                           : DION3_ERR_HIP;
}

static int side_ctx(size_t nev, SideCtx** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DION3_ERR_HIP;
  SideCtx& c = g_side[dev];
  if (!c.side) {
    if (hipStreamCreateWithFlags(&c.side, hipStreamNonBlocking) != hipSuccess) {
      c.side = nullptr;
      return DION3_ERR_HIP;
    }
    c.gen = ++g_side_gen;
  }
  // the overlap streams are created when a step first needs one (run_step):
  // a process holds only the kind its steps use
  while (c.ev.size() < nev) {
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return DION3_ERR_HIP;
    c.ev.push_back(e);
  }
  *out = &c;
  return DION3_OK;
}
// Destroys the library streams and events of every device (see dion3_release).
int release_step_resources() {
  std::lock_guard<std::mutex> lock(g_side_mu);
  int st = DION3_OK;
  int prev = -1;
  for (int d = 0; d < kMaxDevices; ++d) {
    SideCtx& c = g_side[d];
    if (!c.side && !c.mem && !c.mem_all && c.ev.empty()) continue;
    if (prev < 0 && hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (hipSetDevice(d) != hipSuccess) { st = DION3_ERR_HIP; continue; }
    // the streams' queued work completes before they are destroyed
    for (hipStream_t* q : {&c.side, &c.mem, &c.mem_all}) {
      if (!*q) continue;
      if (hipStreamSynchronize(*q) != hipSuccess || hipStreamDestroy(*q) != hipSuccess) st = DION3_ERR_HIP;
      *q = nullptr;
    }
    for (hipEvent_t e : c.ev)
      if (hipEventDestroy(e) != hipSuccess) st = DION3_ERR_HIP;
    c.ev.clear();
  }
  if (prev >= 0 && hipSetDevice(prev) != hipSuccess) st = DION3_ERR_HIP;
  return st;
}
}  // namespace dion3

using namespace dion3;

extern "C" size_t dion3_step_workspace_bytes(int n_groups, const dion3_group* groups, const int* k,
                                             const dion3_ns_params* p) {
  Plan P;
  if (!make_plan(n_groups, groups, k, p, P)) return 0;
  return P.bytes();
}

// V == nullptr: Muon flavour; otherwise NorMuon with the per-line second
// moments V[i] ([batch][n] fp32 per group), beta2 and nm_eps.
static int run_step(int n_groups, const dion3_group* groups, void* const* W, void* const* M,
                    const void* const* G, const int* k, int32_t* const* idx,
                    const dion3_ns_params* p, float eta, float wd, float mu, void* ws,
                    size_t ws_bytes, void* stream, bool deferred, bool has_prev,
                    float* const* V = nullptr, float beta2 = 0.f, float nm_eps = 0.f) {
  Plan P;
  if (!W || !M || !G || !idx || !make_plan(n_groups, groups, k, p, P)) return DION3_ERR_INVALID_ARG;
  for (int i = 0; i < n_groups; ++i)
    if (!W[i] || !M[i] || !G[i] || !idx[i] || (V && !V[i])) return DION3_ERR_INVALID_ARG;
  if (V && (!(beta2 >= 0.f && beta2 <= 1.f) || !(nm_eps >= 0.f))) return DION3_ERR_INVALID_ARG;
  if (!ws || ws_bytes < P.bytes()) return DION3_ERR_WORKSPACE;
  const int nc = (int)P.classes.size();
  // workspace: top-k partials | per-group selected sums of squares |
  // NorMuon row factors | X0 of alternate classes (the next class is gathered
  // while this one's products run) | outputs of alternate classes (a class's
  // update may still read the previous output) | Newton-Schulz scratch
  char* base = (char*)ws;
  char* rs_ws = base;
  char* sqn_base = rs_ws + P.rowsel;
  char* rsc_base = sqn_base + P.sqn;
  const int nx = nc > 1 ? 2 : 1;
  char* X0 = rsc_base + P.rs;
  char* X0buf[2] = {X0, X0 + (nx - 1) * P.xbuf};
  char* Obuf[2] = {X0 + nx * P.xbuf, X0 + (2 * nx - 1) * P.xbuf};
  char* gws = X0 + 2 * nx * P.xbuf;
  const size_t es = dtype_size(p->ns_dtype);
  hipStream_t s = (hipStream_t)stream;

  // graph capture of the multi-stream step is not supported: refuse before
  // anything is enqueued (a step graph built node by node, graph.hip, is)
  if (!graph_builder()) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) return DION3_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return DION3_ERR_UNSUPPORTED;
  }

  std::lock_guard<std::mutex> lock(g_side_mu);
  SideCtx* ctx = nullptr;
  int st = side_ctx(3 * (size_t)nc + 3, &ctx);
  if (st) return st;
  // The overlapped passes keep half of the units only when they are large:
  // then the products beside them keep the other half (7B set: 26 GB of
  // momentum traffic beside the first class's products, 26.3 against 27.1 ms
  // per step with every unit).  Small passes are better spread over every unit
  // (1B set: 4.8 GB, 2.92 against 3.10 ms).
  double overlapped = 0.0;          // momentum bytes of the classes after the first
  for (int c = 1; c < nc; ++c)
    for (int i : P.classes[c])
      overlapped += 3.0 * (double)dtype_size(groups[i].dtype) * groups[i].rows * groups[i].cols * groups[i].batch;
  const bool masked = overlapped >= kMaskedOverlapBytes;
  if (nc > 1) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DION3_ERR_HIP;
    if (masked && !ctx->mem && make_mem_stream(dev, &ctx->mem) != DION3_OK) {
      ctx->mem = nullptr;
      return DION3_ERR_HIP;
    }
    if (!masked && !ctx->mem_all && hipStreamCreateWithFlags(&ctx->mem_all, hipStreamNonBlocking) != hipSuccess) {
      ctx->mem_all = nullptr;
      return DION3_ERR_HIP;
    }
  }
  hipStream_t side = ctx->side, mem = masked ? ctx->mem : ctx->mem_all;
  hipEvent_t* ev_sel = ctx->ev.data();          // class c selected
  hipEvent_t* ev_ns = ev_sel + nc;              // class c orthogonalised (side stream)
  hipEvent_t* ev_upd = ev_ns + nc;              // class c updated
  hipEvent_t ev_fork = ev_upd[nc];              // first class selected (caller's stream)
  hipEvent_t ev_side_end = ev_upd[nc + 1];      // side stream drained
  hipEvent_t ev_mem_end = ev_upd[nc + 2];       // overlapped stream drained
  // class c's momentum + selection and gather: the caller's stream for the
  // first class, else the overlapped stream; class c's update: the caller's
  // stream for the last class, else the overlapped stream
  auto sel_stream = [&](int c) { return c == 0 ? s : mem; };
  auto upd_stream = [&](int c) { return c == nc - 1 ? s : mem; };
  bool used_side = false, used_mem = false;

  // momentum + selection of class c, then the gather of its selected lines
  // into X0buf[c & 1] (free once class c - 2's Newton-Schulz has ended)
  auto select_and_gather = [&](int c) -> int {
    hipStream_t sc = sel_stream(c);
    const auto& cls = P.classes[c];
    const int kk = k[cls[0]], mm = P.m[cls[0]];
    const size_t slice = (size_t)kk * mm * es;
    int r = DION3_OK;
    for (int i : cls) {
      const dion3_group& gi = groups[i];
      // deferred error feedback: idx[i] holds the previous selection on entry;
      // its decay is applied in this pass, then idx[i] is overwritten
      r = dion3_momentum_rowsel_ef(&gi, M[i], G[i], k[i], idx[i], nullptr, (double*)(sqn_base + P.sqn_off[i]),
                                   deferred && has_prev ? idx[i] : nullptr, k[i], mu, rs_ws, P.rowsel, sc);
      if (r) return r;
    }
    if (c >= 2 && (r = stream_wait(sc, ev_ns[c - 2]))) return r;
    int nb = 0;
    for (int i : cls) {
      const dion3_group& gi = groups[i];
      r = dion3_gather_rows(&gi, M[i], idx[i], kk, (const double*)(sqn_base + P.sqn_off[i]), p->eps,
                            p->ns_dtype, X0buf[c & 1] + nb * slice, sc);
      if (r) return r;
      nb += gi.batch;
    }
    return event_record(ev_sel[c], sc);
  };

  st = select_and_gather(0);
  if (!st && nc > 1) {
    // the overlapped stream starts once the first class is gathered
    st = event_record(ev_fork, s);
    if (!st) st = stream_wait(mem, ev_fork);
    used_mem = used_mem || !st;
  }
  for (int c = 0; c < nc && !st; ++c) {
    const auto& cls = P.classes[c];
    const int kk = k[cls[0]], mm = P.m[cls[0]];
    const size_t slice = (size_t)kk * mm * es;
    char* O = Obuf[c & 1];
    // Newton-Schulz of class c on the side stream
    st = stream_wait(side, ev_sel[c]);
    used_side = used_side || !st;
    // O is rewritten two classes later: wait until that class's update read it
    if (!st && c >= 2) st = stream_wait(side, ev_upd[c - 2]);
    int nb = 0;
    for (int i : cls) nb += groups[i].batch;
    // Muon flavour with deferred decay (the update leaves M alone): the last
    // product updates W itself for row-selected bf16 groups, whose O is then
    // never written or read
    const bool can_fuse = deferred && !V;
    std::vector<FusedSegment> segs;
    FusedUpdate fu{};
    if (can_fuse) {
      int b0 = 0;
      for (int i : cls) {
        const dion3_group& gi = groups[i];
        int gn = 0, gm = 0, gax = 0;
        FusedSegment sg{};
        sg.b0 = b0;
        sg.nb = gi.batch;
        sg.fuse = canonical_dims(&gi, &gn, &gm, &gax) && gax == 0 && gi.dtype == DION3_BF16;
        sg.W = W[i];
        sg.sW = gi.batch_stride;
        sg.wlines = gn;
        sg.idx = idx[i];
        segs.push_back(sg);
        b0 += gi.batch;
      }
      fu.nseg = (int)segs.size();
      fu.seg = segs.data();
      fu.eta = eta;
      fu.u = weight_decay_factor(eta, wd);
      fu.decay = wd != 0.0f;
    }
    // aspect ratio 1: standard Newton-Schulz on the symmetric kernels (fewer
    // launches, equal work); otherwise Gram Newton-Schulz
    FusedUpdate* fup = can_fuse ? &fu : nullptr;
    if (!st) st = mm == kk ? standard_ns_fused(nb, kk, mm, p, X0buf[c & 1], O, gws, P.gram, side, fup)
                           : gram_ns_gathered_fused(nb, kk, mm, p, X0buf[c & 1], O, gws, P.gram, side, fup);
    if (!st) st = event_record(ev_ns[c], side);
    // the next class's momentum and gather go ahead of this class's update
    // on the overlapped stream, so that they run beside these products
    if (!st && c + 1 < nc) st = select_and_gather(c + 1);
    // the update of class c
    hipStream_t uc = upd_stream(c);
    if (!st) st = stream_wait(uc, ev_ns[c]);
    nb = 0;
    int si = 0;
    for (int i : cls) {
      if (st) break;
      const dion3_group& gi = groups[i];
      if (can_fuse && segs[si++].fused) {
        // W's selected lines are updated; weight decay of the others remains
        if (wd != 0.0f) st = decay_unselected(&gi, W[i], idx[i], kk, weight_decay_factor(eta, wd), uc);
        nb += gi.batch;
        continue;
      }
      float* rsc = V ? (float*)(rsc_base + P.rs_off[i]) : nullptr;
      if (V)
        st = dion3_normuon_scale(&gi, idx[i], kk, O + nb * slice, p->ns_dtype, (long long)kk * mm, V[i],
                                 beta2, nm_eps, rsc, uc);
      if (!st)
        st = dion3_apply_rows_scaled(&gi, W[i], deferred ? nullptr : M[i], idx[i], kk, O + nb * slice,
                                     p->ns_dtype, (long long)kk * mm, rsc, eta, wd, mu, uc);
      nb += gi.batch;
    }
    if (!st) st = event_record(ev_upd[c], uc);
  }
  // join: the caller's stream waits for everything enqueued on the library
  // streams (also after an error, so that no such work escapes the call's order)
  auto join = [&](hipStream_t from, hipEvent_t e) {
    const int j = event_record(e, from);
    const int w = j ? j : stream_wait(s, e);
    if (!st) st = w;
  };
  if (used_side) join(side, ev_side_end);
  if (used_mem) join(mem, ev_mem_end);
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

namespace dion3 {
int run_step_deferred(int n_groups, const dion3_group* groups, void* const* W, void* const* M,
                      const void* const* G, const int* k, int32_t* const* idx, int has_prev,
                      const dion3_ns_params* p, float eta, float wd, float mu, void* ws, size_t ws_bytes,
                      void* stream) {
  return run_step(n_groups, groups, W, M, G, k, idx, p, eta, wd, mu, ws, ws_bytes, stream, true,
                  has_prev != 0);
}
}  // namespace dion3

extern "C" int dion3_step_normuon(int n_groups, const dion3_group* groups, void* const* W,
                                  void* const* M, const void* const* G, const int* k,
                                  int32_t* const* idx, float* const* V, int deferred, int has_prev,
                                  const dion3_ns_params* p, float eta, float wd, float mu,
                                  float beta2, float nm_eps, void* ws, size_t ws_bytes, void* stream) {
  if (!V) return DION3_ERR_INVALID_ARG;
  return run_step(n_groups, groups, W, M, G, k, idx, p, eta, wd, mu, ws, ws_bytes, stream,
                  deferred != 0, deferred != 0 && has_prev != 0, V, beta2, nm_eps);
}
