// The whole optimizer step as a HIP graph, built node by node.
//
// Method: "Dion3: Full-Stack Orthogonal Updates", Section 6: the launches of
// a step form the same dependency structure every step, so the pages replay
// one recorded graph per step instead of issuing every launch from the host.
//
// Here the graph is not recorded by stream capture.  The step driver runs
// once with a builder active on this thread: every launch becomes a kernel
// node (hipGraphAddKernelNode, the arguments copied into the node), each
// stream the driver would use stands for a branch, an event record remembers
// a branch's last nodes and an event wait adds them to the waiting branch's
// dependencies.  The graph therefore has exactly the order the streams and
// events give the eager step, and its nodes are the same kernels with the
// same arguments.  The graph is instantiated once; launching it enqueues the
// step on a stream with one call.
#include <algorithm>
#include <map>
#include <vector>

#include "common.h"

namespace dion3 {

struct GraphBuilder {
  hipGraph_t graph = nullptr;
  std::map<hipStream_t, std::vector<hipGraphNode_t>> last;    // per branch: the nodes a new node follows
  std::map<hipEvent_t, std::vector<hipGraphNode_t>> marks;    // per event: the nodes it stands for
  int status = DION3_OK;
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

// Event record / wait of the step driver: HIP calls when launching eagerly,
// dependency bookkeeping while a graph is being built.
int event_record(hipEvent_t e, hipStream_t s) {
  if (GraphBuilder* b = t_builder) {
    b->marks[e] = b->last[s];
    return b->status;
  }
  return hipEventRecord(e, s) == hipSuccess ? DION3_OK : DION3_ERR_HIP;
}

int stream_wait(hipStream_t s, hipEvent_t e) {
  if (GraphBuilder* b = t_builder) {
    std::vector<hipGraphNode_t>& deps = b->last[s];
    for (hipGraphNode_t n : b->marks[e])
      if (std::find(deps.begin(), deps.end(), n) == deps.end()) deps.push_back(n);
    return b->status;
  }
  return hipStreamWaitEvent(s, e, 0) == hipSuccess ? DION3_OK : DION3_ERR_HIP;
}

}  // namespace dion3

using namespace dion3;

struct dion3_graph_s {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

extern "C" int dion3_step_graph_create(int n_groups, const dion3_group* groups, void* const* W,
                                       void* const* M, const void* const* G, const int* k,
                                       int32_t* const* idx, int has_prev, const dion3_ns_params* p,
                                       float eta, float wd, float mu, void* ws, size_t ws_bytes,
                                       dion3_graph* out) {
  if (!out) return DION3_ERR_INVALID_ARG;
  *out = nullptr;
  // the step's own checks, before any HIP call
  if (!W || !M || !G || !idx || !k || n_groups < 1) return DION3_ERR_INVALID_ARG;
  for (int i = 0; i < n_groups; ++i)
    if (!W[i] || !M[i] || !G[i] || !idx[i]) return DION3_ERR_INVALID_ARG;
  const size_t need = dion3_step_workspace_bytes(n_groups, groups, k, p);
  if (!need) return DION3_ERR_INVALID_ARG;
  if (!ws || ws_bytes < need) return DION3_ERR_WORKSPACE;
  GraphBuilder b;
  if (hipGraphCreate(&b.graph, 0) != hipSuccess) return DION3_ERR_HIP;
  // the caller's branch is the null stream's key; the driver's own streams
  // are keys of the other branches
  t_builder = &b;
  int st = run_step_deferred(n_groups, groups, W, M, G, k, idx, has_prev, p, eta, wd, mu, ws, ws_bytes,
                             nullptr);
  t_builder = nullptr;
  if (!st) st = b.status;
  hipGraphExec_t exec = nullptr;
  if (!st && hipGraphInstantiate(&exec, b.graph, nullptr, nullptr, 0) != hipSuccess) st = DION3_ERR_HIP;
  if (st) {
    (void)hipGraphDestroy(b.graph);
    return st;
  }
  dion3_graph_s* g = new dion3_graph_s;
  g->graph = b.graph;
  g->exec = exec;
  *out = g;
  return DION3_OK;
}

extern "C" int dion3_graph_launch(dion3_graph g, void* stream) {
  if (!g || !g->exec) return DION3_ERR_INVALID_ARG;
  return hipGraphLaunch(g->exec, (hipStream_t)stream) == hipSuccess ? DION3_OK : DION3_ERR_HIP;
}

extern "C" int dion3_graph_destroy(dion3_graph g) {
  if (!g) return DION3_OK;
  int st = DION3_OK;
  if (g->exec && hipGraphExecDestroy(g->exec) != hipSuccess) st = DION3_ERR_HIP;
  if (g->graph && hipGraphDestroy(g->graph) != hipSuccess) st = DION3_ERR_HIP;
  delete g;
  return st;
}
