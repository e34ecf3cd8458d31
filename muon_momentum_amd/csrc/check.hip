// Count of non-finite entries of a buffer: the optional finite check of a
// step's tensors.
//
// Method: "Dion3: Full-Stack Orthogonal Updates", Appendix B (Figure 11):
// trained with the Gram iteration in half precision and no restart, the
// iteration's outputs eventually fill with infinities.  Callers that want to
// watch for that failure (or for non-finite gradients) count the NaN and
// +-Inf entries of G, M, O or W with this pass.
//
// One streaming pass: 16-byte loads when the buffer is 16-byte aligned, a
// per-lane count and one atomic add per lane that saw any into the caller's
// 64-bit device counter.
#include "common.h"

namespace dion3 {

// exponent field all ones: infinity or NaN
__device__ __forceinline__ unsigned nonfinite16(uint32_t h, uint32_t mask) { return (h & mask) == mask; }

__global__ __launch_bounds__(256) void count_nonfinite32_kernel(const uint32_t* __restrict__ x, size_t n, bool vec,
                                                                unsigned long long* __restrict__ count) {
  constexpr uint32_t E = 0x7f800000u;
  unsigned c = 0;
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  if (vec) {
    const size_t nv = n / 4;
    for (size_t i = tid; i < nv; i += stride) {
      const uint4 v = ((const uint4*)x)[i];
      c += ((v.x & E) == E) + ((v.y & E) == E) + ((v.z & E) == E) + ((v.w & E) == E);
    }
    for (size_t i = nv * 4 + tid; i < n; i += stride) c += (x[i] & E) == E;
  } else {
    for (size_t i = tid; i < n; i += stride) c += (x[i] & E) == E;
  }
  if (c) atomicAdd(count, (unsigned long long)c);
}

// 16-bit types: the exponent mask is 0x7c00 (fp16) or 0x7f80 (bf16)
__global__ __launch_bounds__(256) void count_nonfinite16_kernel(const uint16_t* __restrict__ x, size_t n, bool vec,
                                                                uint32_t mask, unsigned long long* __restrict__ count) {
  unsigned c = 0;
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  if (vec) {
    const size_t nv = n / 8;
    for (size_t i = tid; i < nv; i += stride) {
      const uint4 v = ((const uint4*)x)[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) c += nonfinite16(w[q] & 0xffffu, mask) + nonfinite16(w[q] >> 16, mask);
    }
    for (size_t i = nv * 8 + tid; i < n; i += stride) c += nonfinite16(x[i], mask);
  } else {
    for (size_t i = tid; i < n; i += stride) c += nonfinite16(x[i], mask);
  }
  if (c) atomicAdd(count, (unsigned long long)c);
}

}  // namespace dion3

using namespace dion3;

extern "C" int dion3_count_nonfinite(const void* x, int dtype, size_t n, unsigned long long* count, void* stream) {
  if (!x || !count || n == 0) return DION3_ERR_INVALID_ARG;
  if (dtype != DION3_F32 && dtype != DION3_F16 && dtype != DION3_BF16) return DION3_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const size_t es = dtype_size(dtype);
  const bool vec = aligned16(x);
  const size_t per_block = 256 * (16 / es);
  const size_t blocks = (n + per_block - 1) / per_block;
  const dim3 grid((unsigned)(blocks < 4096 ? (blocks ? blocks : 1) : 4096));
  TimedLaunch tl("count_nonfinite", s);
  if (dtype == DION3_F32)
    (void)launch(count_nonfinite32_kernel, grid, dim3(256), s, (const uint32_t*)x, n, vec, count);
  else
    (void)launch(count_nonfinite16_kernel, grid, dim3(256), s, (const uint16_t*)x, n, vec,
                 dtype == DION3_F16 ? 0x7c00u : 0x7f80u, count);
  return launch_status();
}
