// The whole optimizer step as HIP graphs, replayed with a few host calls.
//
// Method: "Dion3: Full-Stack Orthogonal Updates", Section 6: the launches of
// a step form the same dependency structure every step, so the pages replay
// one recorded graph per step instead of issuing every launch from the host.
//
// Here nothing is recorded by stream capture.  The step driver runs once
// with a builder active on the calling thread and its launches and event
// operations are collected in program order.  The kernels a stream receives
// between two event operations on that stream form one segment; each segment
// becomes a graph of kernel nodes in a chain (hipGraphAddKernelNode, the
// arguments copied into the node).  A launch of the step then replays the
// program: each segment as one graph launch on its own stream (the caller's
// stream, or the library's streams with their compute-unit masks), and the
// event records and waits between segments as the driver issues them.  So
// the streams, their masks and the cross-stream order are the eager step's,
// and the host issues about a tenth of the eager step's calls.
//
// With DION3_GRAPH_ONE the whole step is one graph instead: each stream of
// the driver is a branch, an event record remembers the branch's last nodes
// and a wait adds them to the waiting branch's dependencies; one host call
// launches it, and HIP schedules the branches without the library's streams.
#include <algorithm>
#include <map>
#include <vector>

#include "common.h"

namespace dion3 {

struct GraphSegment {
  hipStream_t s = nullptr;          // stream key: nullptr for the caller's stream
  hipGraph_t graph = nullptr;
  hipGraphNode_t last = nullptr;    // the chain's last node while the segment is open
  hipGraphExec_t exec = nullptr;
};

struct GraphOp {
  enum Kind { LAUNCH, RECORD, WAIT } kind;
  hipStream_t s;                    // stream key
  hipEvent_t e;                     // RECORD / WAIT
  int seg;                          // LAUNCH
};

struct GraphBuilder {
  // DION3_GRAPH_ONE: one graph for the whole step, each stream a branch
  // (a node follows its branch's last nodes; a wait adds the nodes the event
  // stood for); HIP schedules the branches itself, without the library's
  // streams or their compute-unit masks
  bool one = false;
  hipGraph_t graph = nullptr;
  std::map<hipStream_t, std::vector<hipGraphNode_t>> last;
  std::map<hipEvent_t, std::vector<hipGraphNode_t>> marks;
  // otherwise: segments and the program that replays them
  std::vector<GraphSegment> segs;
  std::vector<GraphOp> ops;
  std::map<hipStream_t, int> open;  // stream key -> its open segment
  int status = DION3_OK;

  // ends the open segment of s: its launch takes this place in the program
  void close(hipStream_t s) {
    auto it = open.find(s);
    if (it == open.end()) return;
    ops.push_back({GraphOp::LAUNCH, s, nullptr, it->second});
    open.erase(it);
  }
  void close_all() {
    while (!open.empty()) close(open.begin()->first);
  }
};

static thread_local GraphBuilder* t_builder = nullptr;

GraphBuilder* graph_builder() { return t_builder; }

int graph_status(GraphBuilder* b) { return b->status; }

int graph_add_kernel(GraphBuilder* b, const void* func, dim3 grid, dim3 block, void** args, hipStream_t s) {
  if (b->status) return b->status;
  hipKernelNodeParams kp = {};
  kp.func = const_cast<void*>(func);
  kp.gridDim = grid;
  kp.blockDim = block;
  kp.sharedMemBytes = 0;
  kp.kernelParams = args;
  kp.extra = nullptr;
  if (b->one) {
    std::vector<hipGraphNode_t>& deps = b->last[s];
    hipGraphNode_t node = nullptr;
    if (hipGraphAddKernelNode(&node, b->graph, deps.empty() ? nullptr : deps.data(), deps.size(), &kp) !=
        hipSuccess) {
      b->status = DION3_ERR_HIP;
      return b->status;
    }
    deps.assign(1, node);
    return DION3_OK;
  }
  auto it = b->open.find(s);
  int si;
  if (it == b->open.end()) {
    GraphSegment g;
    g.s = s;
    if (hipGraphCreate(&g.graph, 0) != hipSuccess) {
      b->status = DION3_ERR_HIP;
      return b->status;
    }
    si = (int)b->segs.size();
    b->segs.push_back(g);
    b->open[s] = si;
  } else {
    si = it->second;
  }
  GraphSegment& g = b->segs[si];
  hipGraphNode_t node = nullptr;
  if (hipGraphAddKernelNode(&node, g.graph, g.last ? &g.last : nullptr, g.last ? 1 : 0, &kp) != hipSuccess) {
    b->status = DION3_ERR_HIP;
    return b->status;
  }
  g.last = node;
  return DION3_OK;
}

// Event record / wait of the step driver: HIP calls when launching eagerly,
// entries of the program while a step graph is being built.
int event_record(hipEvent_t e, hipStream_t s) {
  if (GraphBuilder* b = t_builder) {
    if (b->one) {
      b->marks[e] = b->last[s];
      return b->status;
    }
    b->close(s);
    b->ops.push_back({GraphOp::RECORD, s, e, -1});
    return b->status;
  }
  return hipEventRecord(e, s) == hipSuccess ? DION3_OK : DION3_ERR_HIP;
}

int stream_wait(hipStream_t s, hipEvent_t e) {
  if (GraphBuilder* b = t_builder) {
    if (b->one) {
      std::vector<hipGraphNode_t>& deps = b->last[s];
      for (hipGraphNode_t n : b->marks[e])
        if (std::find(deps.begin(), deps.end(), n) == deps.end()) deps.push_back(n);
      return b->status;
    }
    b->close(s);
    b->ops.push_back({GraphOp::WAIT, s, e, -1});
    return b->status;
  }
  return hipStreamWaitEvent(s, e, 0) == hipSuccess ? DION3_OK : DION3_ERR_HIP;
}

}  // namespace dion3

using namespace dion3;

struct dion3_graph_s {
  std::vector<GraphSegment> segs;   // DION3_GRAPH_ONE: one segment, no program
  std::vector<GraphOp> ops;
  bool one = false;
  int device = 0;
  unsigned gen = 0;                 // generation of the library streams the program names
};

static void destroy_segments(std::vector<GraphSegment>& segs, int* st) {
  for (GraphSegment& g : segs) {
    if (g.exec && hipGraphExecDestroy(g.exec) != hipSuccess && st) *st = DION3_ERR_HIP;
    if (g.graph && hipGraphDestroy(g.graph) != hipSuccess && st) *st = DION3_ERR_HIP;
    g.exec = nullptr;
    g.graph = nullptr;
  }
}

// Builds the graphs of one step: `run` enqueues the step (the driver, with
// this thread's builder active).
template <typename Run>
static int build_step_graph(unsigned flags, dion3_graph* out, Run run) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DION3_ERR_HIP;
  GraphBuilder b;
  b.one = (flags & DION3_GRAPH_ONE) != 0;
  if (b.one) {
    GraphSegment g;
    if (hipGraphCreate(&g.graph, 0) != hipSuccess) return DION3_ERR_HIP;
    b.graph = g.graph;
    b.segs.push_back(g);
  }
  t_builder = &b;
  int st = run();
  t_builder = nullptr;
  b.close_all();
  if (!st) st = b.status;
  for (GraphSegment& g : b.segs) {
    if (st) break;
    if (hipGraphInstantiate(&g.exec, g.graph, nullptr, nullptr, 0) != hipSuccess) {
      g.exec = nullptr;
      st = DION3_ERR_HIP;
    }
  }
  unsigned gen = 0;
  if (!st) {
    std::lock_guard<std::mutex> lock(side_mutex());
    gen = side_generation();
    if (!gen) st = DION3_ERR_HIP;    // the driver created the library streams above
  }
  if (st) {
    destroy_segments(b.segs, nullptr);
    return st;
  }
  dion3_graph_s* g = new dion3_graph_s;
  g->segs = std::move(b.segs);
  g->ops = std::move(b.ops);
  g->one = b.one;
  g->device = dev;
  g->gen = gen;
  *out = g;
  return DION3_OK;
}

// The step's own argument checks that need no HIP call.
static int check_step_args(int n_groups, const dion3_group* groups, void* const* W, void* const* M,
                           const void* const* G, const int* k, int32_t* const* idx, const dion3_ns_params* p,
                           void* ws, size_t ws_bytes) {
  if (!W || !M || !G || !idx || !k || n_groups < 1) return DION3_ERR_INVALID_ARG;
  for (int i = 0; i < n_groups; ++i)
    if (!W[i] || !M[i] || !G[i] || !idx[i]) return DION3_ERR_INVALID_ARG;
  const size_t need = dion3_step_workspace_bytes(n_groups, groups, k, p);
  if (!need) return DION3_ERR_INVALID_ARG;
  if (!ws || ws_bytes < need) return DION3_ERR_WORKSPACE;
  return DION3_OK;
}

extern "C" int dion3_step_graph_create(int n_groups, const dion3_group* groups, void* const* W,
                                       void* const* M, const void* const* G, const int* k,
                                       int32_t* const* idx, int has_prev, const dion3_ns_params* p,
                                       float eta, float wd, float mu, void* ws, size_t ws_bytes,
                                       unsigned flags, dion3_graph* out) {
  if (!out) return DION3_ERR_INVALID_ARG;
  *out = nullptr;
  if (flags & ~(unsigned)DION3_GRAPH_ONE) return DION3_ERR_INVALID_ARG;
  if (int st = check_step_args(n_groups, groups, W, M, G, k, idx, p, ws, ws_bytes)) return st;
  return build_step_graph(flags, out, [&] {
    return run_step_deferred(n_groups, groups, W, M, G, k, idx, has_prev, p, eta, wd, mu, ws, ws_bytes, nullptr);
  });
}

extern "C" int dion3_step_normuon_graph_create(int n_groups, const dion3_group* groups, void* const* W,
                                               void* const* M, const void* const* G, const int* k,
                                               int32_t* const* idx, float* const* V, int has_prev,
                                               const dion3_ns_params* p, float eta, float wd, float mu,
                                               float beta2, float nm_eps, void* ws, size_t ws_bytes,
                                               unsigned flags, dion3_graph* out) {
  if (!out) return DION3_ERR_INVALID_ARG;
  *out = nullptr;
  if (flags & ~(unsigned)DION3_GRAPH_ONE) return DION3_ERR_INVALID_ARG;
  if (int st = check_step_args(n_groups, groups, W, M, G, k, idx, p, ws, ws_bytes)) return st;
  if (!V) return DION3_ERR_INVALID_ARG;
  for (int i = 0; i < n_groups; ++i)
    if (!V[i]) return DION3_ERR_INVALID_ARG;
  return build_step_graph(flags, out, [&] {
    return dion3_step_normuon(n_groups, groups, W, M, G, k, idx, V, 1, has_prev, p, eta, wd, mu, beta2, nm_eps,
                              ws, ws_bytes, nullptr);
  });
}

extern "C" int dion3_graph_launch(dion3_graph g, void* stream) {
  if (!g) return DION3_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DION3_ERR_HIP;
  if (dev != g->device) return DION3_ERR_INVALID_ARG;
  hipStream_t caller = (hipStream_t)stream;
  if (g->one) return hipGraphLaunch(g->segs[0].exec, caller) == hipSuccess ? DION3_OK : DION3_ERR_HIP;
  // the program uses the library's streams and events: the same lock as an
  // eager step, and the streams it was built with must still exist
  std::lock_guard<std::mutex> lock(side_mutex());
  if (side_generation() != g->gen) return DION3_ERR_INVALID_ARG;
  for (const GraphOp& op : g->ops) {
    hipStream_t s = op.s ? op.s : caller;
    hipError_t e = hipSuccess;
    switch (op.kind) {
      case GraphOp::LAUNCH: e = hipGraphLaunch(g->segs[op.seg].exec, s); break;
      case GraphOp::RECORD: e = hipEventRecord(op.e, s); break;
      case GraphOp::WAIT: e = hipStreamWaitEvent(s, op.e, 0); break;
    }
    if (e != hipSuccess) return DION3_ERR_HIP;
  }
  return DION3_OK;
}

extern "C" int dion3_graph_destroy(dion3_graph g) {
  if (!g) return DION3_OK;
  int st = DION3_OK;
  destroy_segments(g->segs, &st);
  delete g;
  return st;
}
