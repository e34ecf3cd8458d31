// Small C entry points: status strings, k = ceil(f n), canonical sizes, and the
// per-launch event timing used by benchmarks.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "common.h"

using namespace dion3;

extern "C" const char* dion3_status_string(int status) {
  switch (status) {
    case DION3_OK: return "ok";
    case DION3_ERR_INVALID_ARG: return "invalid argument";
    case DION3_ERR_UNSUPPORTED: return "unsupported";
    case DION3_ERR_WORKSPACE: return "workspace missing or too small";
    case DION3_ERR_HIP: return "HIP error";
    case DION3_ERR_TOO_LARGE: return "input needs more than the fixed scratch of the no-allocation entry point";
  }
  return "unknown status";
}

// k = ceil(f n) of the exact product ("Dion3: Full-Stack Orthogonal Updates",
// Section 6).  p = fl(f n) and its exact residual e = f n - p (an FMA) decide
// the one case where rounding lands on an integer from above or below.
extern "C" int dion3_k_from_fraction(int n, double f) {
  if (n < 1 || !(f > 0.0) || !(f <= 1.0)) return DION3_ERR_INVALID_ARG;
  const double p = f * (double)n;
  const double e = fma(f, (double)n, -p);
  double c = ceil(p);
  if (c == p && e > 0.0) c += 1.0;
  long long k = (long long)c;
  if (k < 1) k = 1;
  if (k > n) k = n;
  return (int)k;
}

extern "C" int dion3_canonical(const dion3_group* g, int* n, int* m, int* axis) {
  int nn, mm, ax;
  if (!canonical_dims(g, &nn, &mm, &ax)) return DION3_ERR_INVALID_ARG;
  if (n) *n = nn;
  if (m) *m = mm;
  if (axis) *axis = ax;
  return DION3_OK;
}

// ------------------------------------------------------------------ timing
namespace {
struct Timing {
  std::vector<hipEvent_t> ev;     // 2 per launch
  std::vector<const char*> name;
  int cap = 0, used = 0;
  bool open = false;
};
Timing g_timing;
}  // namespace

namespace dion3 {
void timing_begin(const char* name, hipStream_t s) {
  Timing& T = g_timing;
  if (T.cap == 0 || T.used >= T.cap || graph_builder()) return;   // no events inside a step graph
  if (hipEventRecord(T.ev[2 * T.used], s) != hipSuccess) return;
  T.name[T.used] = name;
  T.open = true;
}
void timing_end(hipStream_t s) {
  Timing& T = g_timing;
  if (!T.open) return;
  T.open = false;
  if (hipEventRecord(T.ev[2 * T.used + 1], s) == hipSuccess) ++T.used;
}
}  // namespace dion3

extern "C" int dion3_timing_enable(int max_launches) {
  Timing& T = g_timing;
  for (hipEvent_t e : T.ev) (void)hipEventDestroy(e);
  T.ev.clear();
  T.name.clear();
  T.cap = T.used = 0;
  T.open = false;
  if (max_launches <= 0) return DION3_OK;
  T.ev.resize(2 * (size_t)max_launches);
  T.name.resize(max_launches, nullptr);
  for (auto& e : T.ev)
    if (hipEventCreate(&e) != hipSuccess) return DION3_ERR_HIP;
  T.cap = max_launches;
  return DION3_OK;
}

extern "C" int dion3_timing_report(char* buf, size_t buf_bytes) {
  Timing& T = g_timing;
  if (!buf || buf_bytes == 0) return DION3_ERR_INVALID_ARG;
  std::vector<const char*> names;
  std::vector<double> total;
  std::vector<int> count;
  for (int i = 0; i < T.used; ++i) {
    if (hipEventSynchronize(T.ev[2 * i + 1]) != hipSuccess) return DION3_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, T.ev[2 * i], T.ev[2 * i + 1]) != hipSuccess) return DION3_ERR_HIP;
    size_t j = 0;
    while (j < names.size() && strcmp(names[j], T.name[i]) != 0) ++j;
    if (j == names.size()) {
      names.push_back(T.name[i]);
      total.push_back(0.0);
      count.push_back(0);
    }
    total[j] += ms;
    count[j] += 1;
  }
  T.used = 0;
  size_t off = 0;
  buf[0] = 0;
  for (size_t j = 0; j < names.size(); ++j) {
    const int w = snprintf(buf + off, buf_bytes - off, "%s %d %.6f\n", names[j], count[j], total[j]);
    if (w < 0 || (size_t)w >= buf_bytes - off) return DION3_ERR_INVALID_ARG;
    off += (size_t)w;
  }
  return (int)off;
}

// Releases everything the library created on its own: the whole-step streams
// and event pool of every device and the timing events.  A later call creates
// what it needs again.  Nothing is released that was never created, so a
// process that never used the GPU makes no HIP call here.
extern "C" int dion3_release(void) {
  const int a = release_step_resources();
  const int b = g_timing.cap > 0 || !g_timing.ev.empty() ? dion3_timing_enable(0) : DION3_OK;
  return a ? a : b;
}
