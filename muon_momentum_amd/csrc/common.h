// Internal helpers shared by the HIP sources of libdion3 (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <tuple>
#include <utility>

#include "dion3.h"

namespace dion3 {

typedef _Float16 f16;
typedef uint16_t bf16_t;   // raw bfloat16 bits

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bfx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- rounding
__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even; a NaN keeps its sign and upper payload
// bits with the quiet bit set, i.e. for bit pattern u: (u >> 16) | 0x40 if u
// is a NaN, else (u + 0x7fff + ((u >> 16) & 1)) >> 16.  gfx950's
// v_cvt_pk_bf16_f32 computes exactly this (compared on all 2^32 inputs, in
// the default floating-point mode these kernels run in); the pair form
// converts two values with one instruction.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  const f32x2_hw v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw));
}

// fp64 -> bf16 with a single round-to-nearest-even of the fp64 value.
__device__ __forceinline__ bf16_t f64_to_bf16(double d) {
  uint64_t u = (uint64_t)__double_as_longlong(d);
  const uint32_t E = (uint32_t)((u >> 52) & 0x7ff);
  if (E == 0x7ff) {                                 // inf or NaN
    if (u & 0x000fffffffffffffull) return (bf16_t)(0x7fc0u | ((u >> 48) & 0x8000u));
    return (bf16_t)(0x7f80u | ((u >> 48) & 0x8000u));
  }
  if (E >= 897) {                                   // |d| >= 2^-126: bf16 normal range
    u += (1ull << 44) - 1ull + ((u >> 45) & 1ull);  // round the significand to 8 bits
    u &= ~((1ull << 45) - 1ull);
    const float f = (float)__longlong_as_double((long long)u);   // exact (or inf)
    return (bf16_t)(__float_as_uint(f) >> 16);
  }
  // bf16 subnormal range: quantum 2^-133
  const double q = rint(d * 0x1p133) * 0x1p-133;     // exact scaling, RNE
  return (bf16_t)(__float_as_uint((float)q) >> 16);
}

// ------------------------------------------------------- sorted index sets
// First position in a[0..n) (ascending) whose value is >= v.
__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <typename T> struct Store;
template <> struct Store<float> {
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};
template <> struct Store<f16> {
  __device__ static float to_f32(f16 v) { return (float)v; }
  __device__ static f16 from_f32(float v) { return (f16)v; }
};
template <> struct Store<bf16_t> {
  __device__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// mu * m rounded once to the storage type (the product of an fp32 and a bf16
// value is exact in fp64; one round-to-nearest-even to bf16 follows).
template <typename T> __device__ __forceinline__ T decay_round(float mu, T m);
template <> __device__ __forceinline__ bf16_t decay_round<bf16_t>(float mu, bf16_t m) {
  return f64_to_bf16((double)mu * (double)bf16_to_f32(m));
}
template <> __device__ __forceinline__ float decay_round<float>(float mu, float m) { return mu * m; }

// The fused update of one selected entry of W: w' = round(fp32(a - eta o))
// with a = fp32(u w) when decaying, else w ("Dion3: Full-Stack Orthogonal
// Updates", Section 6: evaluated in fp32, cast back to storage once).  The
// apply pass and the Q X epilogue that fuses it share this definition.
template <typename T>
__device__ __forceinline__ T update_w(T w, float o, float eta, float u, bool decay) {
  float a = Store<T>::to_f32(w);
  if (decay) a = u * a;
  return Store<T>::from_f32(__builtin_fmaf(-eta, o, a));
}

// ------------------------------------------------------------- reductions
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// --------------------------------------------------------------- host side
inline size_t dtype_size(int dt) {
  return dt == DION3_F32 ? 4 : (dt == DION3_F16 || dt == DION3_BF16) ? 2 : 0;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Per-kernel event timing (measurement only; see dion3_timing_enable).
void timing_begin(const char* name, hipStream_t s);
void timing_end(hipStream_t s);

struct TimedLaunch {
  hipStream_t s;
  TimedLaunch(const char* name, hipStream_t st) : s(st) { timing_begin(name, s); }
  ~TimedLaunch() { timing_end(s); }
};

// ------------------------------------------------------------------ launches
// Every kernel of the library goes through launch(): eagerly onto the stream,
// or, while a step graph is being built on this thread (graph.hip), as a
// kernel node of that graph, the stream standing for a branch of it.  The
// arguments are converted to the kernel's parameter types and passed by
// address, the form both hipLaunchKernel and hipGraphAddKernelNode take.
struct GraphBuilder;
GraphBuilder* graph_builder();                 // this thread's builder, or nullptr
int graph_add_kernel(GraphBuilder* b, const void* func, dim3 grid, dim3 block, void** args, hipStream_t s);
int graph_status(GraphBuilder* b);

template <typename... P, typename... A, size_t... I>
inline int launch_args(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, std::index_sequence<I...>,
                       A&&... a) {
  std::tuple<P...> t(static_cast<P>(std::forward<A>(a))...);
  void* args[] = {(void*)&std::get<I>(t)...};
  if (GraphBuilder* b = graph_builder()) return graph_add_kernel(b, (const void*)kernel, grid, block, args, s);
  return hipLaunchKernel((const void*)kernel, grid, block, args, 0, s) == hipSuccess ? DION3_OK : DION3_ERR_HIP;
}
template <typename... P, typename... A>
inline int launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, A&&... a) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  return launch_args(kernel, grid, block, s, std::index_sequence_for<P...>{}, std::forward<A>(a)...);
}

// Status of the launches since the last check (the graph being built, or the
// last HIP error of this thread).
inline int launch_status() {
  if (GraphBuilder* b = graph_builder()) return graph_status(b);
  return hipGetLastError() == hipSuccess ? DION3_OK : DION3_ERR_HIP;
}

inline bool canonical_dims(const dion3_group* g, int* n, int* m, int* axis) {
  if (!g || g->rows <= 0 || g->cols <= 0 || g->batch <= 0) return false;
  if ((long long)g->rows * g->cols > g->batch_stride && g->batch > 1) return false;
  int ax = g->sel_axis;
  if (ax != 0 && ax != 1) {
    if (ax != -1) return false;
    ax = g->rows <= g->cols ? 0 : 1;
  }
  *axis = ax;
  *n = ax == 0 ? g->rows : g->cols;
  *m = ax == 0 ? g->cols : g->rows;
  return true;
}

// Destroys the streams and events the whole-step driver created (step.hip).
int release_step_resources();

// The deferred whole step (step.hip), and the event record / stream wait it
// uses: HIP calls, or graph dependencies while a step graph is built (graph.hip).
int run_step_deferred(int n_groups, const dion3_group* groups, void* const* W, void* const* M,
                      const void* const* G, const int* k, int32_t* const* idx, int has_prev,
                      const dion3_ns_params* p, float eta, float wd, float mu, void* ws, size_t ws_bytes,
                      void* stream);
int event_record(hipEvent_t e, hipStream_t s);
// The lock the step driver holds while it enqueues (step.hip), and the
// generation of the current device's library streams (0: none yet or released).
std::mutex& side_mutex();
unsigned side_generation();

// u = fp32(1 - eta wd): the product is exact in fp64, one rounding to fp32
inline float weight_decay_factor(float eta, float wd) { return (float)(1.0 - (double)eta * (double)wd); }

// The last product of a Newton-Schulz call (O = Q X) with the update of W
// fused into it for some groups of the batch: segment s covers matrices
// [b0, b0 + nb) of the batch, those of one group; `fuse` asks for the fused
// update of that group's W (bf16, rows selected by idx).  The call reports
// per segment whether it fused (else it wrote that segment's O).
struct FusedSegment {
  int b0, nb;
  void* W; long long sW; int wlines; const int32_t* idx;
  bool fuse, fused;
};
struct FusedUpdate {
  int nseg;
  FusedSegment* seg;
  float eta, u; int decay;
};
int gram_ns_gathered_fused(int batch, int k, int m, const dion3_ns_params* p, const void* X0, void* O, void* ws,
                           size_t ws_bytes, void* stream, FusedUpdate* fu);
int standard_ns_fused(int batch, int k, int m, const dion3_ns_params* p, const void* X0, void* O, void* ws,
                      size_t ws_bytes, void* stream, FusedUpdate* fu);
// Weight decay of the lines a step did not select (scatter.hip; W bf16 or fp32).
int decay_unselected(const dion3_group* g, void* W, const int32_t* idx, int k, float u, hipStream_t s);
int stream_wait(hipStream_t s, hipEvent_t e);

// ||M[S,:]||_F^2 of every matrix of a group (scatter.hip); line_ws holds
// [batch][k] fp64 per-line sums.
int selected_sqnorm(const dion3_group* g, int axis, const void* M, const int32_t* idx, int k,
                    double* line_ws, double* sqn, hipStream_t s);

// ------------------------------------------------- GEMM launchers (gemm.hip)
enum GemmOp { OP_SYRK = 0, OP_SQ_ADD = 1, OP_SYM_MUL = 2, OP_GEMM = 3 };

struct GemmArgs {
  int op;
  int dtype;          // operand dtype
  int out_dtype;      // result dtype
  int batch;
  int M, N, K;        // C is M x N; contraction length K
  const void* A; long long lda, sA;
  const void* B; long long ldb, sB;     // B operand (K-contiguous rows, or X for OP_GEMM)
  const void* E; long long lde, sE;     // epilogue operand (beta term), may be null
  void* C; long long ldc, sC;
  float alpha, beta, gamma;
  int reverse = 0;    // visit the batch from its last matrix (tile order only)
  // Q X with the update of W fused into the epilogue (OP_GEMM, large tiles,
  // bf16 W): row r of matrix b's result, rounded to out_dtype, updates row
  // idx[b][r] of W's matrix b (wlines rows of N elements, matrix stride sW)
  // with update_w; C receives only the rows whose index is out of range.
  void* W = nullptr; long long sW = 0; int wlines = 0; const int32_t* idx = nullptr;
  float eta = 0.f, u = 1.f; int decay = 0;
};

int launch_gemm(const GemmArgs& a, hipStream_t s);
// Whether launch_gemm runs `a` on the large-tile kernel, and whether it can
// fuse the update into it (large tiles, 16-bit result, 16-byte aligned W rows).
bool gemm_large_tile(const GemmArgs& a);
bool gemm_fused_update_ok(const GemmArgs& a);

}  // namespace dion3
