// Momentum accumulation fused with the selection keys, and deterministic top-k.
//
// Method: "Dion3: Full-Stack Orthogonal Updates", Section 6: the momentum is
// accumulated as M <- M + G before the update is formed (the mu-damping of the
// selected rows happens after the update), and the k = ceil(f n) rows of
// largest l1 norm are selected; rows or columns, whichever dimension is smaller.
//
// Kernel 1 (HBM-bound, one pass over M and G): M <- round(M + G) with the sum
// formed in fp32 and rounded once to the storage type, and per canonical line
// the fp64 sums of |M| (the key) and M^2 (for the Frobenius norm of the
// selected submatrix).  Row selection: one wave per row, lane-sequential
// accumulation then a butterfly reduction.  Column selection: a work-group
// owns 512 columns x 512 rows; each lane owns 8 columns; the four waves are
// combined in a fixed order and written as per-chunk partial sums.
// Kernel 2 (one work-group per matrix): sums the partials in chunk order,
// radix-selects the k-th largest key on its 64-bit pattern (non-negative
// doubles order like their bit patterns; NaN is mapped to +inf), breaks ties
// toward lower indices with an ordered prefix count, and compacts the selected
// indices in ascending order.  Every reduction has a fixed order, so results
// are bitwise reproducible.
#include <mutex>

#include "common.h"

namespace dion3 {

constexpr int kColBlock = 512;     // columns per work-group (column selection)
constexpr int kChunkRows = 512;    // rows per work-group (column selection)
constexpr int kTopkThreads = 1024;
constexpr int kTopkPer = 32;       // keys per thread -> n <= 32768
constexpr int kRowsPerWave = 2;

template <typename T> struct Vec;
template <> struct Vec<bf16_t> { static constexpr int N = 8; };
template <> struct Vec<float> { static constexpr int N = 4; };

// 16-byte streaming accesses of the momentum pass: every byte of M and G is
// touched once per step, so the loads and stores are non-temporal and do not
// displace anything worth keeping in the caches.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(void* p, uint4 v) {
  u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (u32x4*)p);
}

template <typename T>
__device__ __forceinline__ T add_round(T m, T g) {
  return Store<T>::from_f32(Store<T>::to_f32(m) + Store<T>::to_f32(g));
}

// M + G, after the pending error-feedback decay when `dec`: round(round(mu M) + G)
template <typename T>
__device__ __forceinline__ T accumulate(T m, T g, bool dec, float mu) {
  return add_round(dec ? decay_round<T>(mu, m) : m, g);
}

// ------------------------------------------------------------- row selection
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void momentum_rows_kernel(
    T* __restrict__ M, const T* __restrict__ G, int rows, int cols, long long bstride,
    double* __restrict__ pkey, double* __restrict__ psq, const int32_t* __restrict__ pidx, int pk,
    float mu) {
  constexpr int V = Vec<T>::N;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = (blockIdx.x * 4 + wave) * kRowsPerWave;
  // rows selected by the previous step (decay still pending): one search for
  // the wave's first row, then a walk along the ascending selection
  const int32_t* pb = pidx ? pidx + (long long)b * pk : nullptr;
  int pos = pidx ? lower_bound_i32(pb, pk, r0) : 0;
  for (int r = r0; r < r0 + kRowsPerWave && r < rows; ++r) {
    bool dec = false;
    if (pidx) {
      while (pos < pk && pb[pos] < r) ++pos;
      dec = pos < pk && pb[pos] == r;
    }
    T* mr = M + b * bstride + (long long)r * cols;
    const T* gr = G + b * bstride + (long long)r * cols;
    double s1 = 0.0, s2 = 0.0;
    if (VEC) {
      constexpr int U = 4;
      for (int c0 = lane * V; c0 < cols; c0 += 64 * V * U) {
        uint4 vm[U], vg[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * 64 * V;
          if (c < cols) {
            vm[u] = ld_stream(mr + c);
            vg[u] = ld_stream(gr + c);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * 64 * V;
          if (c < cols) {
            union { uint4 v; T e[16 / sizeof(T)]; } um, ug;
            um.v = vm[u];
            ug.v = vg[u];
#pragma unroll
            for (int e = 0; e < (int)(16 / sizeof(T)); ++e) {
              const T x = accumulate(um.e[e], ug.e[e], dec, mu);
              um.e[e] = x;
              const double d = (double)Store<T>::to_f32(x);
              s1 += fabs(d);
              s2 += d * d;
            }
            st_stream(mr + c, um.v);
          }
        }
      }
    } else {
      for (int c = lane; c < cols; c += 64) {
        const T x = accumulate(mr[c], gr[c], dec, mu);
        mr[c] = x;
        const double d = (double)Store<T>::to_f32(x);
        s1 += fabs(d);
        s2 += d * d;
      }
    }
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    if (lane == 0) {
      pkey[(long long)b * rows + r] = s1;
      psq[(long long)b * rows + r] = s2;
    }
  }
}

// ---------------------------------------------------------- column selection
// grid: x = column blocks of 512, y = row chunks of 256, z = batch.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void momentum_cols_kernel(
    T* __restrict__ M, const T* __restrict__ G, int rows, int cols, long long bstride,
    double* __restrict__ pkey, double* __restrict__ psq, const int32_t* __restrict__ pidx, int pk,
    float mu) {
  constexpr int E = 8;   // columns per lane
  __shared__ double red[2][4][kColBlock];
  __shared__ uint32_t dmask[kColBlock / 32];   // columns of this block selected last step
  const int b = blockIdx.z, chunk = blockIdx.y, nchunks = gridDim.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // VEC: 8 contiguous columns per lane; otherwise columns lane + 64 e.
  auto col_of = [&](int e) { return blockIdx.x * kColBlock + (VEC ? lane * E + e : lane + 64 * e); };
  const int cb = blockIdx.x * kColBlock;
  if (threadIdx.x < kColBlock / 32) dmask[threadIdx.x] = 0u;
  __syncthreads();
  if (pidx) {
    const int32_t* pb = pidx + (long long)b * pk;
    const int lo = lower_bound_i32(pb, pk, cb), hi = lower_bound_i32(pb, pk, cb + kColBlock);
    for (int t = lo + threadIdx.x; t < hi; t += 256) {
      const unsigned lc = (unsigned)(pb[t] - cb);
      if (lc < (unsigned)kColBlock) atomicOr(&dmask[lc >> 5], 1u << (lc & 31));
    }
  }
  __syncthreads();
  bool dec[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int lc = col_of(e) - cb;
    dec[e] = (dmask[lc >> 5] >> (lc & 31)) & 1u;
  }
  double s1[E], s2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) s1[e] = s2[e] = 0.0;
  const int rbeg = chunk * kChunkRows;
  const int rend = min(rbeg + kChunkRows, rows);
  T* Mb = M + b * bstride;
  const T* Gb = G + b * bstride;
#pragma unroll 4
  for (int r = rbeg + wave; r < rend; r += 4) {
    T* mr = Mb + (long long)r * cols;
    const T* gr = Gb + (long long)r * cols;
    if (VEC) {
      const int c = col_of(0);
      if (c < cols) {
        union { uint4 v[E * sizeof(T) / 16]; T e[E]; } um, ug;
#pragma unroll
        for (int w = 0; w < (int)(E * sizeof(T) / 16); ++w) {
          um.v[w] = ld_stream(mr + c + w * (16 / sizeof(T)));
          ug.v[w] = ld_stream(gr + c + w * (16 / sizeof(T)));
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const T x = accumulate(um.e[e], ug.e[e], dec[e], mu);
          um.e[e] = x;
          const double d = (double)Store<T>::to_f32(x);
          s1[e] += fabs(d);
          s2[e] += d * d;
        }
#pragma unroll
        for (int w = 0; w < (int)(E * sizeof(T) / 16); ++w)
          st_stream(mr + c + w * (16 / sizeof(T)), um.v[w]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int c = col_of(e);
        if (c < cols) {
          const T x = accumulate(mr[c], gr[c], dec[e], mu);
          mr[c] = x;
          const double d = (double)Store<T>::to_f32(x);
          s1[e] += fabs(d);
          s2[e] += d * d;
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int lc = VEC ? lane * E + e : lane + 64 * e;
    red[0][wave][lc] = s1[e];
    red[1][wave][lc] = s2[e];
  }
  __syncthreads();
  for (int lc = threadIdx.x; lc < kColBlock; lc += 256) {
    const int c = blockIdx.x * kColBlock + lc;
    if (c < cols) {
      const double k1 = ((red[0][0][lc] + red[0][1][lc]) + red[0][2][lc]) + red[0][3][lc];
      const double k2 = ((red[1][0][lc] + red[1][1][lc]) + red[1][2][lc]) + red[1][3][lc];
      const long long o = ((long long)b * nchunks + chunk) * cols + c;
      pkey[o] = k1;
      psq[o] = k2;
    }
  }
}

// ------------------------------------------------------------------ top-k
// Exclusive prefix count of `flag` over the block in thread order, and total.
__device__ __forceinline__ int block_prefix(bool flag, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long mask = __ballot(flag);
  const int lanepre = __popcll(mask & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = __popcll(mask);
  __syncthreads();
  int pre = 0, tot = 0;
  const int nw = blockDim.x >> 6;
  for (int w = 0; w < nw; ++w) {
    const int v = wsum[w];
    pre += w < wave ? v : 0;
    tot += v;
  }
  __syncthreads();
  total = tot;
  return pre + lanepre;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const double* __restrict__ pkey, const double* __restrict__ psq, int n, int nchunks, int k,
    int32_t* __restrict__ idx, double* __restrict__ keys_out, double* __restrict__ sel_sqnorm) {
  __shared__ unsigned hist[256];
  __shared__ int wsum[kTopkThreads / 64];
  __shared__ int s_digit, s_krem;
  __shared__ double red[kTopkThreads];

  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const double* pk = pkey + (long long)b * nchunks * n;
  const double* ps = psq + (long long)b * nchunks * n;
  const int per = (n + kTopkThreads - 1) / kTopkThreads;

  uint64_t u[kTopkPer];
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) {
    u[j] = 0;
    const int i = t + kTopkThreads * j;
    if (j < per && i < n) {
      double v = 0.0;
      for (int c = 0; c < nchunks; ++c) v += pk[(long long)c * n + i];
      if (keys_out) keys_out[(long long)b * n + i] = v;
      u[j] = v != v ? 0x7ff0000000000000ull : (uint64_t)__double_as_longlong(v);
    }
  }

  // radix select of the k-th largest key, 8 bits at a time from the top
  uint64_t prefix = 0, pmask = 0;
  int krem = k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int h = t; h < 256; h += kTopkThreads) hist[h] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTopkPer; ++j) {
      const int i = t + kTopkThreads * j;
      if (j < per && i < n && (u[j] & pmask) == prefix)
        atomicAdd(&hist[(unsigned)(u[j] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (t < 64) {
      // wave 0: lane l owns digits 255 - 4l .. 252 - 4l; a suffix scan over
      // the lanes finds the digit where the count from the top reaches krem
      const int d0 = 255 - 4 * t;
      const int c0 = (int)hist[d0], c1 = (int)hist[d0 - 1], c2 = (int)hist[d0 - 2], c3 = (int)hist[d0 - 3];
      const int mine = c0 + c1 + c2 + c3;
      int incl = mine;                                   // inclusive prefix over lanes 0..t
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (t >= off) incl += v;
      }
      const int before = incl - mine;
      const unsigned long long hit = __ballot(incl >= krem);
      const int lane_hit = hit ? __ffsll((long long)hit) - 1 : 63;
      if (t == lane_hit) {
        int acc = before, d = d0;
        const int cs[4] = {c0, c1, c2, c3};
        int q = 0;
        for (; q < 3; ++q) {
          if (acc + cs[q] >= krem) break;
          acc += cs[q];
        }
        d = d0 - q;
        s_digit = d;
        s_krem = krem - acc;
      }
    }
    __syncthreads();
    prefix |= (uint64_t)s_digit << shift;
    pmask |= 255ull << shift;
    krem = s_krem;
    __syncthreads();
  }
  const uint64_t thr = prefix;   // the k-th largest key; take `krem` of the equal ones

  int eq_base = 0, sel_base = 0;
  double sq = 0.0;
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) {
    if (j >= per) break;           // uniform over the block: barriers stay matched
    const int i = t + kTopkThreads * j;
    const bool valid = i < n;
    const bool eq = valid && u[j] == thr;
    const bool gt = valid && u[j] > thr;
    int eq_tot, sel_tot;
    const int eq_pre = block_prefix(eq, wsum, eq_tot) + eq_base;
    const bool sel = gt || (eq && eq_pre < krem);
    const int pos = block_prefix(sel, wsum, sel_tot) + sel_base;
    if (sel && pos < k) {
      idx[(long long)b * k + pos] = i;
      double s = 0.0;
      for (int c = 0; c < nchunks; ++c) s += ps[(long long)c * n + i];
      sq += s;
    }
    eq_base += eq_tot;
    sel_base += sel_tot;
  }
  if (sel_sqnorm) {
    red[t] = sq;
    __syncthreads();
    for (int w = kTopkThreads / 2; w >= 1; w >>= 1) {
      if (t < w) red[t] += red[t + w];
      __syncthreads();
    }
    if (t == 0) sel_sqnorm[b] = red[0];
  }
}

// ------------------------------------------------------------------ host
static int nchunks_for(int axis, int rows) {
  return axis == 0 ? 1 : (rows + kChunkRows - 1) / kChunkRows;
}

template <typename T>
static void launch_momentum(const dion3_group* g, int axis, void* M, const void* G,
                            double* pkey, double* psq, const int32_t* pidx, int pk, float mu,
                            hipStream_t s) {
  constexpr int V = Vec<T>::N;
  const bool vec = g->cols % V == 0 && (g->batch == 1 || g->batch_stride % V == 0) &&
                   aligned16(M) && aligned16(G);
  TimedLaunch tl("momentum_keys", s);
  if (axis == 0) {
    dim3 grid((g->rows + 4 * kRowsPerWave - 1) / (4 * kRowsPerWave), g->batch);
    if (vec)
      (void)launch((momentum_rows_kernel<T, true>), grid, dim3(256), s, (T*)M, (const T*)G, g->rows, g->cols, g->batch_stride, pkey, psq, pidx, pk, mu);
    else
      (void)launch((momentum_rows_kernel<T, false>), grid, dim3(256), s, (T*)M, (const T*)G, g->rows, g->cols, g->batch_stride, pkey, psq, pidx, pk, mu);
  } else {
    const bool vec8 = vec && g->cols % 8 == 0;
    dim3 grid((g->cols + kColBlock - 1) / kColBlock, nchunks_for(1, g->rows), g->batch);
    if (vec8)
      (void)launch((momentum_cols_kernel<T, true>), grid, dim3(256), s, (T*)M, (const T*)G, g->rows, g->cols, g->batch_stride, pkey, psq, pidx, pk, mu);
    else
      (void)launch((momentum_cols_kernel<T, false>), grid, dim3(256), s, (T*)M, (const T*)G, g->rows, g->cols, g->batch_stride, pkey, psq, pidx, pk, mu);
  }
}

}  // namespace dion3

using namespace dion3;

extern "C" size_t dion3_rowsel_workspace_bytes(const dion3_group* g) {
  int n, m, axis;
  if (!canonical_dims(g, &n, &m, &axis)) return 0;
  const size_t nch = (size_t)nchunks_for(axis, g->rows);
  const size_t bytes = 2 * (size_t)g->batch * nch * (size_t)n * sizeof(double);
  return bytes < 256 ? 256 : bytes;
}

extern "C" int dion3_momentum_rowsel_ef(const dion3_group* g, void* M, const void* G, int k,
                                        int32_t* idx, double* keys, double* sel_sqnorm,
                                        const int32_t* prev_idx, int prev_k, float mu,
                                        void* ws, size_t ws_bytes, void* stream) {
  int n, m, axis;
  if (!canonical_dims(g, &n, &m, &axis)) return DION3_ERR_INVALID_ARG;
  if (!M || !G || !idx || k < 1 || k > n) return DION3_ERR_INVALID_ARG;
  if (prev_idx && (prev_k < 1 || prev_k > n)) return DION3_ERR_INVALID_ARG;
  if (g->dtype != DION3_F32 && g->dtype != DION3_BF16) return DION3_ERR_INVALID_ARG;
  if (n > kTopkThreads * kTopkPer) return DION3_ERR_UNSUPPORTED;
  const size_t need = dion3_rowsel_workspace_bytes(g);
  if (!ws || ws_bytes < need) return DION3_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int nch = nchunks_for(axis, g->rows);
  double* pkey = (double*)ws;
  double* psq = pkey + (size_t)g->batch * nch * n;
  if (g->dtype == DION3_BF16)
    launch_momentum<bf16_t>(g, axis, M, G, pkey, psq, prev_idx, prev_k, mu, s);
  else
    launch_momentum<float>(g, axis, M, G, pkey, psq, prev_idx, prev_k, mu, s);
  int st = launch_status();
  if (st) return st;
  {
    TimedLaunch tl("topk_select", s);
    (void)launch(topk_kernel, dim3(g->batch), dim3(kTopkThreads), s, pkey, psq, n, nch, k, idx, keys, sel_sqnorm);
  }
  return launch_status();
}

extern "C" int dion3_momentum_rowsel(const dion3_group* g, void* M, const void* G, int k,
                                     int32_t* idx, double* keys, double* sel_sqnorm,
                                     void* ws, size_t ws_bytes, void* stream) {
  return dion3_momentum_rowsel_ef(g, M, G, k, idx, keys, sel_sqnorm, nullptr, 0, 0.f, ws, ws_bytes,
                                  stream);
}

// ------------------------------------------- the entry point that allocates nothing
// The top-k partial sums of dion3_momentum_rowsel_noalloc live in this fixed
// array instead of a caller's workspace.  Each GPU holds its own copy until
// the process ends; host code never passes the array's name to a kernel (on
// the host it is only a stand-in), but the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device on the first call there.  Every partial sum is written before it is
// read, so nothing needs clearing between calls.
static __device__ __align__(256) char scratch[DION3_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kScratchDevices];   // per device: its copy of `scratch`
}  // namespace

static int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return DION3_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DION3_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return DION3_OK;
}

extern "C" int dion3_momentum_rowsel_noalloc(const dion3_group* g, void* M, const void* G, int k,
                                             int32_t* idx, double* keys, double* sel_sqnorm,
                                             const int32_t* prev_idx, int prev_k, float mu,
                                             void* stream) {
  int n, m, axis;
  if (!canonical_dims(g, &n, &m, &axis)) return DION3_ERR_INVALID_ARG;
  if (!M || !G || !idx || k < 1 || k > n) return DION3_ERR_INVALID_ARG;
  if (prev_idx && (prev_k < 1 || prev_k > n)) return DION3_ERR_INVALID_ARG;
  if (g->dtype != DION3_F32 && g->dtype != DION3_BF16) return DION3_ERR_INVALID_ARG;
  if (n > kTopkThreads * kTopkPer) return DION3_ERR_UNSUPPORTED;
  if (dion3_rowsel_workspace_bytes(g) > (size_t)DION3_NOALLOC_SCRATCH_BYTES) return DION3_ERR_TOO_LARGE;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st) return st;
  return dion3_momentum_rowsel_ef(g, M, G, k, idx, keys, sel_sqnorm, prev_idx, prev_k, mu, ws,
                                  (size_t)DION3_NOALLOC_SCRATCH_BYTES, stream);
}
