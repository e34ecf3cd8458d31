// NorMuon flavour of the update.
//
// Method: "Dion3: Full-Stack Orthogonal Updates", Section 2 (NorMuon divides
// each row of the orthogonalised update by the root of that row's second
// moment, an exponential moving average over steps, and rescales the update so
// that its Frobenius norm is Muon's) and Section 6 (the flavour updates the
// second moments of the selected rows only and rescales O before the fused
// weight update; the normalisation runs in fp32).  Per matrix, for the k
// selected lines with Newton-Schulz output rows O_i (length m):
//   q_i = (sum_j O_ij^2) / m
//   v_i <- beta2 v_i + (1 - beta2) q_i          (fp32, stored per line)
//   d_i = 1 / (sqrt(v_i) + eps)
//   r   = ||O||_F / ||diag(d) O||_F             (1 if the update is zero)
//   row_scale_i = d_i r
// The update then uses row_scale_i O_ij in place of O_ij.
//
// Kernel 1: one wave per selected row, fp32 sum of squares (lane-sequential,
// then a fixed butterfly).  Kernel 2: one work-group per matrix, the moments,
// the row factors and the rescale, with the two Frobenius sums in fp64 in a
// fixed order.  Both are deterministic.
#include "common.h"

namespace dion3 {

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <typename TO, bool VEC>
__global__ __launch_bounds__(256) void row_sqsum_kernel(const TO* __restrict__ O, long long ostride,
                                                        int k, int m, float* __restrict__ out) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = blockIdx.x * 4 + wave;
  if (i >= k) return;
  const TO* o = O + b * ostride + (long long)i * m;
  float acc = 0.f;
  if (VEC) {
    // 16-byte loads: 16 / sizeof(TO) elements per lane per step
    constexpr int E = 16 / (int)sizeof(TO);
    for (int c = lane * E; c < m; c += 64 * E) {
      union { uint4 v; TO e[E]; } u;
      u.v = *(const uint4*)(o + c);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float x = Store<TO>::to_f32(u.e[e]);
        acc = __builtin_fmaf(x, x, acc);
      }
    }
  } else {
    for (int c = lane; c < m; c += 64) {
      const float x = Store<TO>::to_f32(o[c]);
      acc = __builtin_fmaf(x, x, acc);
    }
  }
  acc = wave_sum_f(acc);
  if (lane == 0) out[(long long)b * k + i] = acc;
}

// rs holds the rows' sums of squares on entry and their factors on exit.
__global__ __launch_bounds__(256) void normuon_scale_kernel(const int32_t* __restrict__ idx, int k, int m,
                                                            float* __restrict__ V, int nlines, float beta2,
                                                            float eps, float* __restrict__ rs) {
  __shared__ double red[2][256];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const float om = 1.f - beta2;
  const float fm = (float)m;
  float* rb = rs + (long long)b * k;
  const int32_t* ib = idx + (long long)b * k;
  float* vb = V + (long long)b * nlines;
  double so = 0.0, sh = 0.0;
  for (int i = t; i < k; i += 256) {
    const float s = rb[i];
    const int r = ib[i];
    float vn = 0.f;
    if (r >= 0 && r < nlines) {
      vn = __builtin_fmaf(beta2, vb[r], om * (s / fm));
      vb[r] = vn;
    }
    const float d = 1.f / (sqrtf(vn) + eps);
    rb[i] = d;
    so += (double)s;
    sh += (double)d * (double)d * (double)s;
  }
  red[0][t] = so;
  red[1][t] = sh;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (t < w) {
      red[0][t] += red[0][t + w];
      red[1][t] += red[1][t + w];
    }
    __syncthreads();
  }
  const double r = red[1][0] > 0.0 ? sqrt(red[0][0] / red[1][0]) : 1.0;
  for (int i = t; i < k; i += 256) rb[i] = (float)((double)rb[i] * r);
}

template <typename TO>
static void launch_normuon(const dion3_group* g, int n, int m, const int32_t* idx, int k, const void* O,
                           long long ostride, float* V, float beta2, float eps, float* rs, hipStream_t s) {
  TimedLaunch tl("normuon_scale", s);
  const bool vec = m % (16 / (int)sizeof(TO)) == 0 && aligned16(O) &&
                   (g->batch == 1 || ostride % (16 / (int)sizeof(TO)) == 0);
  dim3 grid((k + 3) / 4, g->batch);
  if (vec)
    (void)launch((row_sqsum_kernel<TO, true>), grid, dim3(256), s, (const TO*)O, ostride, k, m, rs);
  else
    (void)launch((row_sqsum_kernel<TO, false>), grid, dim3(256), s, (const TO*)O, ostride, k, m, rs);
  (void)launch(normuon_scale_kernel, dim3(g->batch), dim3(256), s, idx, k, m, V, n, beta2, eps, rs);
}

}  // namespace dion3

using namespace dion3;

extern "C" int dion3_normuon_scale(const dion3_group* g, const int32_t* idx, int k, const void* O,
                                   int o_dtype, long long o_stride, float* V, float beta2, float eps,
                                   float* row_scale, void* stream) {
  int n, m, axis;
  if (!canonical_dims(g, &n, &m, &axis)) return DION3_ERR_INVALID_ARG;
  if (!idx || !O || !V || !row_scale || k < 1 || k > n) return DION3_ERR_INVALID_ARG;
  if (g->batch > 1 && o_stride < (long long)k * m) return DION3_ERR_INVALID_ARG;
  if (!(beta2 >= 0.f && beta2 <= 1.f) || !(eps >= 0.f)) return DION3_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (o_dtype == DION3_F16)
    launch_normuon<f16>(g, n, m, idx, k, O, o_stride, V, beta2, eps, row_scale, s);
  else if (o_dtype == DION3_F32)
    launch_normuon<float>(g, n, m, idx, k, O, o_stride, V, beta2, eps, row_scale, s);
  else
    return DION3_ERR_INVALID_ARG;
  return launch_status();
}
