// Gather of the selected lines into the Newton-Schulz input, and the fused
// update of W and M.
//
// Method: "Dion3: Full-Stack Orthogonal Updates".
//   Section 2: the Newton-Schulz input is normalised by its Frobenius norm so
//   that every singular value lies in [0, 1].
//   Section 6: W[S,:] <- W[S,:] - eta O with weight decay (if on) applied to
//   all rows first; the whole update is evaluated in fp32 and cast back to the
//   storage type once (the pages fuse it for this reason); error feedback
//   multiplies only the selected rows of M by mu.
//
// Row selection gathers and scatters whole rows (one wave per row, 16-byte
// vectors).  Column selection goes through a 64 x 64 LDS tile so that the
// canonical [k][m] buffers are read and written along m while the stored
// matrix is addressed at the selected columns of each row.
#include "common.h"

namespace dion3 {

template <typename T> struct Pack8;   // 8 elements as whole 16-byte vectors
template <> struct Pack8<bf16_t> { union U { uint4 v[1]; bf16_t e[8]; }; };
template <> struct Pack8<f16> { union U { uint4 v[1]; f16 e[8]; }; };
template <> struct Pack8<float> { union U { uint4 v[2]; float e[8]; }; };

template <typename T>
__device__ __forceinline__ void load8(typename Pack8<T>::U& u, const T* p) {
  // every byte these passes touch is touched once: non-temporal accesses
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int w = 0; w < (int)(8 * sizeof(T) / 16); ++w) {
    const v4u x = __builtin_nontemporal_load((const v4u*)p + w);
    u.v[w] = make_uint4(x.x, x.y, x.z, x.w);
  }
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const typename Pack8<T>::U& u) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int w = 0; w < (int)(8 * sizeof(T) / 16); ++w) {
    const v4u x = {u.v[w].x, u.v[w].y, u.v[w].z, u.v[w].w};
    __builtin_nontemporal_store(x, (v4u*)p + w);
  }
}

__device__ __forceinline__ float nscale(const double* sqn, int b, float eps) {
  return (float)(1.0 / (sqrt(sqn[b]) + (double)eps));
}

// ----------------------------------------------------------------- gather
template <typename TS, typename TX, bool VEC>
__global__ __launch_bounds__(256) void gather_rows_kernel(
    const TS* __restrict__ M, long long bstride, int nlines, int cols, const int32_t* __restrict__ idx,
    int k, const double* __restrict__ sqn, float eps, TX* __restrict__ X) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = blockIdx.x * 4 + wave;
  if (i >= k) return;
  const float sc = nscale(sqn, b, eps);
  const int r = idx[(long long)b * k + i];
  if (r < 0 || r >= nlines) return;
  const TS* src = M + b * bstride + (long long)r * cols;
  TX* dst = X + ((long long)b * k + i) * cols;
  if (VEC) {
    // U chunks of 512 elements per wave in flight: all loads first, then stores
    constexpr int U = 4;
    for (int c0 = lane * 8; c0 < cols; c0 += 64 * 8 * U) {
      typename Pack8<TS>::U a[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 + u * 512 < cols) load8<TS>(a[u], src + c0 + u * 512);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c0 + u * 512 < cols) {
          typename Pack8<TX>::U o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o.e[e] = Store<TX>::from_f32(Store<TS>::to_f32(a[u].e[e]) * sc);
          store8<TX>(dst + c0 + u * 512, o);
        }
      }
    }
  } else {
    for (int c = lane; c < cols; c += 64)
      dst[c] = Store<TX>::from_f32(Store<TS>::to_f32(src[c]) * sc);
  }
}

// X[b][i][j] = M[b][j][idx[i]] * scale;  grid (m/64, k/64, batch)
template <typename TS, typename TX>
__global__ __launch_bounds__(256) void gather_cols_kernel(
    const TS* __restrict__ M, long long bstride, int rows, int cols, const int32_t* __restrict__ idx,
    int k, const double* __restrict__ sqn, float eps, TX* __restrict__ X) {
  __shared__ float tile[64][65];
  const int b = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  const int il = t & 63;
  const float sc = nscale(sqn, b, eps);
  int col = i0 + il < k ? idx[(long long)b * k + i0 + il] : -1;
  if (col >= cols) col = -1;
  const TS* Mb = M + b * bstride;
#pragma unroll 4
  for (int s = 0; s < 16; ++s) {
    const int jj = (t >> 6) + 4 * s;
    const int j = j0 + jj;
    float v = 0.f;
    if (col >= 0 && j < rows) v = Store<TS>::to_f32(Mb[(long long)j * cols + col]);
    tile[il][jj] = v * sc;
  }
  __syncthreads();
#pragma unroll 4
  for (int s = 0; s < 16; ++s) {
    const int il2 = (t >> 6) + 4 * s;
    const int jl = t & 63;
    const int i = i0 + il2, j = j0 + jl;
    if (i < k && j < rows) X[((long long)b * k + i) * rows + j] = Store<TX>::from_f32(tile[il2][jl]);
  }
}

// ------------------------------------------- Frobenius norm of the selection
// Sum of squares of every selected line, in fp64, one wave per line; lanes
// accumulate in a fixed order and a butterfly combines them.  Rows: the line
// is contiguous; columns: lane l reads rows l, l + 64, ... of the column.
template <typename TS>
__global__ __launch_bounds__(256) void line_sqsum_kernel(
    const TS* __restrict__ M, long long bstride, int rows, int cols, int axis,
    const int32_t* __restrict__ idx, int k, double* __restrict__ out) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = blockIdx.x * 4 + wave;
  if (i >= k) return;
  const int nlines = axis == 0 ? rows : cols;
  const int r = idx[(long long)b * k + i];
  double s = 0.0;
  if (r >= 0 && r < nlines) {
    const TS* Mb = M + b * bstride;
    if (axis == 0) {
      const TS* src = Mb + (long long)r * cols;
      for (int c = lane; c < cols; c += 64) {
        const double v = (double)Store<TS>::to_f32(src[c]);
        s += v * v;
      }
    } else {
      for (int j = lane; j < rows; j += 64) {
        const double v = (double)Store<TS>::to_f32(Mb[(long long)j * cols + r]);
        s += v * v;
      }
    }
  }
  s = wave_sum(s);
  if (lane == 0) out[(long long)b * k + i] = s;
}

// Per matrix, the sum of its k line sums: thread t adds lines t, t + 256, ...
// in order, then a fixed tree over the threads.
__global__ __launch_bounds__(256) void sum_lines_kernel(const double* __restrict__ in, int k,
                                                        double* __restrict__ out) {
  __shared__ double red[256];
  const int b = blockIdx.x, t = threadIdx.x;
  double s = 0.0;
  for (int i = t; i < k; i += 256) s += in[(long long)b * k + i];
  red[t] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) out[b] = red[0];
}

// ------------------------------------------------------------------ apply
template <typename TS, typename TO, bool VEC>
__global__ __launch_bounds__(256) void apply_rows_kernel(
    TS* __restrict__ W, TS* __restrict__ M, long long bstride, int nlines, int cols,
    const int32_t* __restrict__ idx, int k, const TO* __restrict__ O, long long ostride,
    const float* __restrict__ rs, float eta, float u_, int decay, float mu) {
  // W == nullptr: decay M only; M == nullptr: update W only (decay deferred);
  // rs (may be NULL): a factor per row of O (NorMuon), one fp32 product
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = blockIdx.x * 4 + wave;
  if (i >= k) return;
  const int r = idx[(long long)b * k + i];
  if (r < 0 || r >= nlines) return;
  const bool dw = W != nullptr, dm = M != nullptr;
  TS* w = dw ? W + b * bstride + (long long)r * cols : nullptr;
  TS* mm = dm ? M + b * bstride + (long long)r * cols : nullptr;
  const TO* o = dw ? O + b * ostride + (long long)i * cols : nullptr;
  const float f = (dw && rs) ? rs[(long long)b * k + i] : 1.f;   // x * 1 is exact
  if (VEC) {
    // U chunks of 512 elements per wave in flight: all loads first, then stores
    constexpr int U = 4;
    for (int c0 = lane * 8; c0 < cols; c0 += 64 * 8 * U) {
      typename Pack8<TS>::U vw[U], vm[U];
      typename Pack8<TO>::U vo[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * 512;
        if (c < cols) {
          if (dw) { load8<TS>(vw[u], w + c); load8<TO>(vo[u], o + c); }
          if (dm) load8<TS>(vm[u], mm + c);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * 512;
        if (c < cols) {
          if (dw) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              vw[u].e[e] = update_w<TS>(vw[u].e[e], Store<TO>::to_f32(vo[u].e[e]) * f, eta, u_, decay != 0);
            store8<TS>(w + c, vw[u]);
          }
          if (dm) {
#pragma unroll
            for (int e = 0; e < 8; ++e) vm[u].e[e] = decay_round<TS>(mu, vm[u].e[e]);
            store8<TS>(mm + c, vm[u]);
          }
        }
      }
    }
  } else {
    for (int c = lane; c < cols; c += 64) {
      if (dw) w[c] = update_w<TS>(w[c], Store<TO>::to_f32(o[c]) * f, eta, u_, decay != 0);
      if (dm) mm[c] = decay_round<TS>(mu, mm[c]);
    }
  }
}

// W[b][j][idx[i]] and M[b][j][idx[i]] for the canonical O[b][i][j]; grid (m/64, k/64, batch).
// W == nullptr: decay M only; M == nullptr: update W only (decay deferred).
template <typename TS, typename TO>
__global__ __launch_bounds__(256) void apply_cols_kernel(
    TS* __restrict__ W, TS* __restrict__ M, long long bstride, int rows, int cols,
    const int32_t* __restrict__ idx, int k, const TO* __restrict__ O, long long ostride,
    const float* __restrict__ rs, float eta, float u, int decay, float mu) {
  __shared__ float tile[64][65];
  const int b = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  const bool dw = W != nullptr, dm = M != nullptr;
  if (dw) {
    const TO* Ob = O + b * ostride;
#pragma unroll 4
    for (int s = 0; s < 16; ++s) {
      const int il2 = (t >> 6) + 4 * s;
      const int jl = t & 63;
      const int i = i0 + il2, j = j0 + jl;
      const float f = (rs && i < k) ? rs[(long long)b * k + i] : 1.f;   // x * 1 is exact
      tile[il2][jl] = (i < k && j < rows) ? Store<TO>::to_f32(Ob[(long long)i * rows + j]) * f : 0.f;
    }
  }
  __syncthreads();
  const int il = t & 63;
  const int col = i0 + il < k ? idx[(long long)b * k + i0 + il] : -1;
  if (col < 0 || col >= cols) return;
  TS* Wb = dw ? W + b * bstride : nullptr;
  TS* Mb = dm ? M + b * bstride : nullptr;
#pragma unroll 4
  for (int s = 0; s < 16; ++s) {
    const int jj = (t >> 6) + 4 * s;
    const int j = j0 + jj;
    if (j < rows) {
      const long long off = (long long)j * cols + col;
      if (dw) Wb[off] = update_w<TS>(Wb[off], tile[il][jj], eta, u, decay != 0);
      if (dm) Mb[off] = decay_round<TS>(mu, Mb[off]);
    }
  }
}

// Weight decay of the unselected lines, W <- round(fp32(u w)) (only when wd != 0).
template <typename TS>
__global__ __launch_bounds__(256) void decay_unselected_kernel(
    TS* __restrict__ W, long long bstride, int rows, int cols, int axis, int n,
    const int32_t* __restrict__ idx, int k, float u) {
  __shared__ uint32_t selmap[1024];   // n <= 32768 bits
  const int b = blockIdx.y;
  const int32_t* ib = idx + (long long)b * k;
  for (int w = threadIdx.x; w < (n + 31) / 32; w += 256) selmap[w] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < k; i += 256)
    if (ib[i] >= 0 && ib[i] < n) atomicOr(&selmap[ib[i] >> 5], 1u << (ib[i] & 31));
  __syncthreads();
  TS* Wb = W + b * bstride;
  // a work-group handles 8 stored rows
  for (int rr = 0; rr < 8; ++rr) {
    const int r = blockIdx.x * 8 + rr;
    if (r >= rows) break;
    if (axis == 0 && ((selmap[r >> 5] >> (r & 31)) & 1u)) continue;
    TS* wr = Wb + (long long)r * cols;
    for (int c = threadIdx.x; c < cols; c += 256) {
      if (axis == 1 && ((selmap[c >> 5] >> (c & 31)) & 1u)) continue;
      wr[c] = Store<TS>::from_f32(u * Store<TS>::to_f32(wr[c]));
    }
  }
}

// ------------------------------------------------------------------ host
template <typename TS, typename TX>
static void launch_gather(const dion3_group* g, int axis, int n, int m, const void* M,
                          const int32_t* idx, int k, const double* sqn, float eps, void* X,
                          hipStream_t s) {
  TimedLaunch tl("gather_scale", s);
  if (axis == 0) {
    const bool vec = m % 8 == 0 && (g->batch == 1 || g->batch_stride % 8 == 0) && aligned16(M) &&
                     aligned16(X);
    dim3 grid((k + 3) / 4, g->batch);
    if (vec)
      (void)launch((gather_rows_kernel<TS, TX, true>), grid, dim3(256), s, (const TS*)M, g->batch_stride, n, m, idx, k, sqn, eps, (TX*)X);
    else
      (void)launch((gather_rows_kernel<TS, TX, false>), grid, dim3(256), s, (const TS*)M, g->batch_stride, n, m, idx, k, sqn, eps, (TX*)X);
  } else {
    dim3 grid((m + 63) / 64, (k + 63) / 64, g->batch);
    (void)launch((gather_cols_kernel<TS, TX>), grid, dim3(256), s, (const TS*)M, g->batch_stride, g->rows, g->cols, idx, k, sqn, eps, (TX*)X);
  }
}

template <typename TS, typename TO>
static void launch_apply(const dion3_group* g, int axis, int n, int m, void* W, void* M,
                         const int32_t* idx, int k, const void* O, long long ostride, const float* rs,
                         float eta, float wd, float mu, hipStream_t s) {
  const float u = weight_decay_factor(eta, wd);
  const int decay = wd != 0.0f;
  TimedLaunch tl(W ? "apply_update" : "decay_rows", s);
  if (decay && W) {
    dim3 grid((g->rows + 7) / 8, g->batch);
    (void)launch((decay_unselected_kernel<TS>), grid, dim3(256), s, (TS*)W, g->batch_stride, g->rows, g->cols, axis, n, idx, k, u);
  }
  if (axis == 0) {
    const bool vec = m % 8 == 0 && (g->batch == 1 || (g->batch_stride % 8 == 0 && ostride % 8 == 0)) &&
                     aligned16(W) && aligned16(M) && aligned16(O);
    dim3 grid((k + 3) / 4, g->batch);
    if (vec)
      (void)launch((apply_rows_kernel<TS, TO, true>), grid, dim3(256), s, (TS*)W, (TS*)M, g->batch_stride, n, m, idx, k, (const TO*)O, ostride, rs, eta, u, decay, mu);
    else
      (void)launch((apply_rows_kernel<TS, TO, false>), grid, dim3(256), s, (TS*)W, (TS*)M, g->batch_stride, n, m, idx, k, (const TO*)O, ostride, rs, eta, u, decay, mu);
  } else {
    dim3 grid((m + 63) / 64, (k + 63) / 64, g->batch);
    (void)launch((apply_cols_kernel<TS, TO>), grid, dim3(256), s, (TS*)W, (TS*)M, g->batch_stride, g->rows, g->cols, idx, k, (const TO*)O, ostride, rs, eta, u, decay, mu);
  }
}

int decay_unselected(const dion3_group* g, void* W, const int32_t* idx, int k, float u, hipStream_t s) {
  int n, m, axis;
  if (!canonical_dims(g, &n, &m, &axis) || !W || !idx || k < 1 || k > n || n > 32768) return DION3_ERR_INVALID_ARG;
  TimedLaunch tl("apply_update", s);
  dim3 grid((g->rows + 7) / 8, g->batch);
  if (g->dtype == DION3_BF16)
    (void)launch((decay_unselected_kernel<bf16_t>), grid, dim3(256), s, (bf16_t*)W, g->batch_stride, g->rows, g->cols, axis, n, idx, k, u);
  else if (g->dtype == DION3_F32)
    (void)launch((decay_unselected_kernel<float>), grid, dim3(256), s, (float*)W, g->batch_stride, g->rows, g->cols, axis, n, idx, k, u);
  else
    return DION3_ERR_INVALID_ARG;
  return launch_status();
}

// ||M[S,:]||_F^2 per matrix into sqn[batch] (fp64), with line_ws [batch][k]
// fp64 holding the per-line sums.  Arguments are validated by the caller.
int selected_sqnorm(const dion3_group* g, int axis, const void* M, const int32_t* idx, int k,
                    double* line_ws, double* sqn, hipStream_t s) {
  TimedLaunch tl("selected_norm", s);
  dim3 grid((k + 3) / 4, g->batch);
  if (g->dtype == DION3_BF16)
    (void)launch((line_sqsum_kernel<bf16_t>), grid, dim3(256), s, (const bf16_t*)M, g->batch_stride, g->rows, g->cols, axis, idx, k, line_ws);
  else if (g->dtype == DION3_F32)
    (void)launch((line_sqsum_kernel<float>), grid, dim3(256), s, (const float*)M, g->batch_stride, g->rows, g->cols, axis, idx, k, line_ws);
  else
    return DION3_ERR_INVALID_ARG;
  (void)launch(sum_lines_kernel, dim3(g->batch), dim3(256), s, (const double*)line_ws, k, sqn);
  return launch_status();
}

}  // namespace dion3

using namespace dion3;

extern "C" int dion3_gather_rows(const dion3_group* g, const void* M, const int32_t* idx, int k,
                                 const double* sel_sqnorm, float eps, int x_dtype, void* X,
                                 void* stream) {
  int n, m, axis;
  if (!canonical_dims(g, &n, &m, &axis)) return DION3_ERR_INVALID_ARG;
  if (!M || !idx || !sel_sqnorm || !X || k < 1 || k > n || !(eps >= 0.f)) return DION3_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (g->dtype == DION3_BF16 && x_dtype == DION3_F16)
    launch_gather<bf16_t, f16>(g, axis, n, m, M, idx, k, sel_sqnorm, eps, X, s);
  else if (g->dtype == DION3_BF16 && x_dtype == DION3_F32)
    launch_gather<bf16_t, float>(g, axis, n, m, M, idx, k, sel_sqnorm, eps, X, s);
  else if (g->dtype == DION3_F32 && x_dtype == DION3_F32)
    launch_gather<float, float>(g, axis, n, m, M, idx, k, sel_sqnorm, eps, X, s);
  else if (g->dtype == DION3_F32 && x_dtype == DION3_F16)
    launch_gather<float, f16>(g, axis, n, m, M, idx, k, sel_sqnorm, eps, X, s);
  else
    return DION3_ERR_INVALID_ARG;
  return launch_status();
}

extern "C" int dion3_apply_rows_scaled(const dion3_group* g, void* W, void* M, const int32_t* idx,
                                       int k, const void* O, int o_dtype, long long o_stride,
                                       const float* row_scale, float eta, float wd, float mu,
                                       void* stream) {
  int n, m, axis;
  if (!canonical_dims(g, &n, &m, &axis)) return DION3_ERR_INVALID_ARG;
  if (!W || !idx || !O || k < 1 || k > n) return DION3_ERR_INVALID_ARG;   // M, row_scale may be NULL
  if (g->batch > 1 && o_stride < (long long)k * m) return DION3_ERR_INVALID_ARG;
  if (n > 32768) return DION3_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const float* rs = row_scale;
  if (g->dtype == DION3_BF16 && o_dtype == DION3_F16)
    launch_apply<bf16_t, f16>(g, axis, n, m, W, M, idx, k, O, o_stride, rs, eta, wd, mu, s);
  else if (g->dtype == DION3_BF16 && o_dtype == DION3_F32)
    launch_apply<bf16_t, float>(g, axis, n, m, W, M, idx, k, O, o_stride, rs, eta, wd, mu, s);
  else if (g->dtype == DION3_F32 && o_dtype == DION3_F32)
    launch_apply<float, float>(g, axis, n, m, W, M, idx, k, O, o_stride, rs, eta, wd, mu, s);
  else if (g->dtype == DION3_F32 && o_dtype == DION3_F16)
    launch_apply<float, f16>(g, axis, n, m, W, M, idx, k, O, o_stride, rs, eta, wd, mu, s);
  else
    return DION3_ERR_INVALID_ARG;
  return launch_status();
}

extern "C" int dion3_apply_rows(const dion3_group* g, void* W, void* M, const int32_t* idx, int k,
                                const void* O, int o_dtype, long long o_stride, float eta, float wd,
                                float mu, void* stream) {
  return dion3_apply_rows_scaled(g, W, M, idx, k, O, o_dtype, o_stride, nullptr, eta, wd, mu, stream);
}

extern "C" int dion3_decay_rows(const dion3_group* g, void* M, const int32_t* idx, int k, float mu,
                                void* stream) {
  int n, m, axis;
  if (!canonical_dims(g, &n, &m, &axis)) return DION3_ERR_INVALID_ARG;
  if (!M || !idx || k < 1 || k > n) return DION3_ERR_INVALID_ARG;
  if (n > 32768) return DION3_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  if (g->dtype == DION3_BF16)
    launch_apply<bf16_t, bf16_t>(g, axis, n, m, nullptr, M, idx, k, nullptr, 0, nullptr, 0.f, 0.f, mu, s);
  else if (g->dtype == DION3_F32)
    launch_apply<float, float>(g, axis, n, m, nullptr, M, idx, k, nullptr, 0, nullptr, 0.f, 0.f, mu, s);
  else
    return DION3_ERR_INVALID_ARG;
  return launch_status();
}
