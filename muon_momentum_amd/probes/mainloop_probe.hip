// Resource probe of the large-tile GEMM's main loop (not part of the library).
//
// One stage of the 256 x 256 kernel (gemm.hip) per work-group of 4 waves, one
// work-group per compute unit (the stage ring takes the whole 160 KB of LDS):
//   DMA   8 `buffer_load_dwordx4 ... lds` per wave: 32 KB of operands into the
//         ring buffer 4 stages ahead, waited for 2 stages ahead (vmcnt 16);
//         either as the kernel loads them (16 rows x 64 bytes per instruction)
//         or as whole 128-byte lines (8 rows x 128 bytes: a layout with two
//         stages' K per row);
//   READ  16 `ds_read_b128` fragment reads per wave (64 KB per unit);
//   MFMA  32 `v_mfma_f32_32x32x16_f16` per wave (128 x 128 per wave);
// interleaved as in the kernel (MFMA, read, MFMA, read, MFMA, DMA, MFMA; the
// loads of the steady state issued without a test) and ended by a barrier.
// Each mode runs a subset, so the cycles per stage of each resource alone can
// be set against the combination, and the clock (shader cycles over wall
// time) shows what the MFMAs cost in power: the operands are random finite
// fp16 values or zeros, and come either from one 4 MB panel pair read by
// every work-group (resident in each XCD's L2 after the first touch) or from
// a 4 MB pair per work-group (HBM).  Results are discarded; every access
// stays inside the buffers below.
//
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 \
//     -Xclang -target-feature -Xclang -packed-fp32-ops \
//     muon_momentum_amd/probes/mainloop_probe.hip -o mainloop_probe && ./mainloop_probe
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <type_traits>
#include <vector>

typedef int int4v __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                      \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                  \
      exit(1);                                                                        \
    }                                                                                 \
  } while (0)

// raw buffer resource of `bytes` bytes at `base` (out-of-range lanes read 0)
__device__ __forceinline__ int4v make_rsrc(const void* base, long long bytes) {
  const unsigned long long a = (unsigned long long)base;
  int4v r;
  r.x = __builtin_amdgcn_readfirstlane((int)(a & 0xffffffffu));
  r.y = __builtin_amdgcn_readfirstlane((int)(a >> 32) & 0xffff);
  r.z = __builtin_amdgcn_readfirstlane(bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
  r.w = 0x00020000;
  return r;
}
// 64 lanes x 16 bytes into LDS at `lds` + 16 x lane (the caller waits: vmcnt)
__device__ __forceinline__ void lds_dma16(const int4v& rsrc, unsigned lds, int voffset, int soffset) {
  const int m0 = __builtin_amdgcn_readfirstlane((int)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m0), "v"(voffset), "s"(rsrc), "s"(soffset) : "memory", "m0");
}
// two finite fp16 values of magnitude below 2 from a hash of k
__host__ __device__ __forceinline__ unsigned mix(unsigned x) {
  x ^= x >> 13;
  x *= 0x5bd1e995u;
  x ^= x >> 15;
  return x & 0xbbffbbffu;
}
__device__ __forceinline__ int swz32(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }
__device__ __forceinline__ u32x4v lds_read16(unsigned addr) {
  return *(const __attribute__((address_space(3))) u32x4v*)(uintptr_t)addr;
}

constexpr int kDma = 1, kRead = 2, kMfma = 4, kWide = 8;

template <int MODE>
__global__ __launch_bounds__(256, 1) void stage_probe(const char* src, long long wg_stride, int ld_bytes, int S,
                                                      bool random, unsigned long long* cyc, float* sink) {
  constexpr bool DMA = MODE & kDma, RD = MODE & kRead, MF = MODE & kMfma, WIDE = MODE & kWide;
  __shared__ __attribute__((aligned(1024))) char smem[5 * 32768];
  const unsigned lds0 = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)smem;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const char* base = src + (long long)blockIdx.x * wg_stride;
  // A: rows 0..255 of the pair, B: rows 256..511; ld_bytes per row, S stages of 64 bytes
  const int4v ra = make_rsrc(base, 256LL * ld_bytes);
  const int4v rb = make_rsrc(base + 256LL * ld_bytes, 256LL * ld_bytes);
  // narrow (the kernel's layout): an instruction covers 16 rows x 64 bytes,
  // half of each 128-byte line.  WIDE: 8 rows x 128 bytes, whole lines, as a
  // layout holding two stages' K per row would load them (stage s: rows
  // 128 (s mod 2) .. + 127 of each operand, bytes 128 (s / 2) .. + 127)
  const int va = WIDE ? (8 * wave + (lane >> 3)) * ld_bytes + ((lane & 7) << 4)
                      : (16 * wave + (lane >> 2)) * ld_bytes + (((lane & 3) ^ (lane >> 4)) << 4);
  const int ka = (WIDE ? 32 : 64) * ld_bytes;
  auto dma = [&](int ls, int b, int x) {
    const unsigned buf = lds0 + (unsigned)(b * 32768);
    const int q = x & 3;
    if (WIDE) {
      const int off = (ls & 1) * 128 * ld_bytes + (ls >> 1) * 128 + q * ka;
      if (x < 4) lds_dma16(ra, buf + (32 * q + 8 * wave) * 128, va, off);
      else lds_dma16(rb, buf + 16384 + (32 * q + 8 * wave) * 128, va, off);
    } else {
      if (x < 4) lds_dma16(ra, buf + (64 * q + 16 * wave) * 64, va, ls * 64 + q * ka);
      else lds_dma16(rb, buf + 16384 + (64 * q + 16 * wave) * 64, va, ls * 64 + q * ka);
    }
  };
  floatx16 acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};
  u32x4v fa[2][4], fb[2][4];
  // fragments for the modes without LDS reads: the same kind of values
  auto rnd = [&](unsigned k) { return mix(k * 2654435761u + threadIdx.x * 40503u + 12345u); };
  for (int h = 0; h < 2; ++h)
    for (int i = 0; i < 4; ++i)
      for (int e = 0; e < 4; ++e) {
        fa[h][i][e] = random ? rnd(16 * h + 4 * i + e) : 0u;
        fb[h][i][e] = random ? rnd(100 + 16 * h + 4 * i + e) : 0u;
      }
  const unsigned long long t0 = __builtin_readcyclecounter();
  if (DMA) {
    for (int g = 0; g < 4 && g < S; ++g)
      for (int x = 0; x < 8; ++x) dma(g, g, x);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  int bcur = 0;
  int g = 0;
  // one stage; ISS: the stage 4 ahead exists (its loads are issued without a
  // test, as in the kernel's steady state)
  auto stage = [&](auto iss_c) {
    constexpr bool ISS = decltype(iss_c)::value;
    const int ib = bcur == 0 ? 4 : bcur - 1;          // buffer of stage g + 4
#pragma unroll
    for (int gx = 0; gx < 8; ++gx) {
      const int st = gx / 4, x = gx % 4;
      u32x4v(&ca)[4] = fa[st];
      u32x4v(&cb)[4] = fb[st];
      u32x4v(&na)[4] = fa[st ^ 1];
      u32x4v(&nb)[4] = fb[st ^ 1];
      const unsigned buf = lds0 + (unsigned)(bcur * 32768);
      auto rd = [&](int h) {
        if (!RD) return;
        if (x < 2)
          nb[2 * x + h] = lds_read16(buf + 16384 + swz32(wn * 128 + (2 * x + h) * 32 + (lane & 31), 2 * (st ^ 1) + (lane >> 5)));
        else
          na[2 * x - 4 + h] = lds_read16(buf + swz32(wm * 128 + (2 * x - 4 + h) * 32 + (lane & 31), 2 * (st ^ 1) + (lane >> 5)));
      };
      auto mm = [&](int jj) {
        if (!MF) return;
        acc[x][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, cb[jj]),
                                                            __builtin_bit_cast(half8, ca[x]), acc[x][jj], 0, 0, 0);
      };
      __builtin_amdgcn_sched_barrier(0);
      mm(0);
      __builtin_amdgcn_sched_barrier(0);
      rd(0);
      __builtin_amdgcn_sched_barrier(0);
      mm(1);
      __builtin_amdgcn_sched_barrier(0);
      rd(1);
      __builtin_amdgcn_sched_barrier(0);
      mm(2);
      __builtin_amdgcn_sched_barrier(0);
      if (DMA && ISS) dma(g + 4, ib, gx);
      __builtin_amdgcn_sched_barrier(0);
      mm(3);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (DMA) {
      if (ISS) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");   // stage g + 2 landed
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    asm volatile("s_barrier" ::: "memory");
    bcur = bcur == 4 ? 0 : bcur + 1;
    ++g;
  };
  for (int t = 0; t < S - 4; ++t) stage(std::true_type{});
  for (int t = S - 4; t < S; ++t) stage(std::false_type{});
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
  const unsigned long long t1 = __builtin_readcyclecounter();
  float s = 0.f;
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) s += acc[i][j][0] + acc[i][j][15];
  for (int h = 0; h < 2; ++h)
    for (int i = 0; i < 4; ++i) s += (float)(fa[h][i].x ^ fb[h][i].w);
  if (s == 1234.5f) sink[0] = s;
  if (threadIdx.x == 0) cyc[blockIdx.x] = t1 - t0;
}

__global__ void fill_random(unsigned* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = mix((unsigned)i * 2654435761u + 777u);
}

template <int MODE>
static void run(const char* name, const char* src, long long wg_stride, int ld_bytes, int S, int grid,
                bool random, unsigned long long* cyc, float* sink) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  stage_probe<MODE><<<grid, 256>>>(src, wg_stride, ld_bytes, S, random, cyc, sink);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  float best = 1e9f;
  for (int r = 0; r < 5; ++r) {
    CHECK(hipEventRecord(e0));
    stage_probe<MODE><<<grid, 256>>>(src, wg_stride, ld_bytes, S, random, cyc, sink);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (ms < best) best = ms;
  }
  std::vector<unsigned long long> h(grid);
  CHECK(hipMemcpy(h.data(), cyc, grid * sizeof(unsigned long long), hipMemcpyDeviceToHost));
  double avg = 0, mx = 0;
  for (auto v : h) { avg += (double)v; if (v > mx) mx = (double)v; }
  avg /= grid;
  const double secs = best * 1e-3;
  printf("%-10s work-groups %3d: %7.1f us  cycles/stage %5.0f (max %5.0f)  clock %.2f GHz  LDS fill %6.2f TB/s  MFMA %5.0f TFLOP/s\n",
         name, grid, best * 1e3, avg / S, mx / S, avg / secs * 1e-9,
         (MODE & kDma) ? (double)grid * S * 32768 / secs * 1e-12 : 0.0,
         (MODE & kMfma) ? (double)grid * S * 4 * 32 * 32768 / secs * 1e-12 : 0.0);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

int main() {
  const int S = 128;                       // stages (K = 4096)
  const int ld = S * 64;                   // bytes per operand row
  const long long pair = 512LL * ld;       // A and B panels of one work-group: 4 MB
  const int maxg = 256;
  char* src = nullptr;
  CHECK(hipMalloc(&src, pair * maxg));
  unsigned long long* cyc = nullptr;
  CHECK(hipMalloc(&cyc, maxg * sizeof(unsigned long long)));
  float* sink = nullptr;
  CHECK(hipMalloc(&sink, sizeof(float)));
  for (int random = 1; random >= 0; --random) {
    if (random) {
      fill_random<<<4096, 256>>>((unsigned*)src, (size_t)(pair * maxg / 4));
      CHECK(hipGetLastError());
    } else {
      CHECK(hipMemset(src, 0, pair * maxg));
    }
    CHECK(hipDeviceSynchronize());
    for (int shared = 1; shared >= 0; --shared) {
      printf("# %s operands: %s\n", random ? "random fp16" : "zero",
             shared ? "one 4 MB panel pair read by every work-group (L2-resident)"
                    : "a 4 MB panel pair per work-group (HBM)");
      const long long stride = shared ? 0 : pair;
      for (int grid : {256, 176}) {
        if (!shared && grid != 256) continue;
        run<kMfma>("mfma", src, stride, ld, S, grid, random, cyc, sink);
        run<kRead | kMfma>("read+mfma", src, stride, ld, S, grid, random, cyc, sink);
        run<kDma>("dma", src, stride, ld, S, grid, random, cyc, sink);
        run<kDma | kRead>("dma+read", src, stride, ld, S, grid, random, cyc, sink);
        run<kDma | kMfma>("dma+mfma", src, stride, ld, S, grid, random, cyc, sink);
        run<kDma | kRead | kMfma>("all", src, stride, ld, S, grid, random, cyc, sink);
        if (shared && grid == 256) {
          run<kDma | kWide>("dma-wide", src, stride, ld, S, grid, random, cyc, sink);
          run<kDma | kMfma | kWide>("wide+mfma", src, stride, ld, S, grid, random, cyc, sink);
          run<kDma | kRead | kMfma | kWide>("wide+all", src, stride, ld, S, grid, random, cyc, sink);
        }
      }
    }
  }
  CHECK(hipFree(src));
  CHECK(hipFree(cyc));
  CHECK(hipFree(sink));
  return 0;
}
