// MFMA GEMM kernels for gfx950: the symmetric products of Gram Newton-Schulz
// (lower-triangle tiles, mirrored write-back, diagonal tiles written once) and
// the rectangular Q X multiply.
//
// Method: "Dion3: Full-Stack Orthogonal Updates", Section 5 (symmetric GEMM:
// a triangular tile scheduler over the lower triangle including the diagonal,
// and an epilogue that writes every off-diagonal tile to its transposed place
// as well) and Appendix C (diagonal tiles are written only once).
//
// Layout: a work-group computes a BM x BN tile of C with 4 waves in a 2 x 2
// arrangement.  Operand tiles are staged in LDS in a K-contiguous layout,
// 128 bytes of K per row per stage, split in 16-byte chunks whose position is
// XOR-swizzled by (row mod 8) so that 32 lanes reading one chunk column hit
// distinct banks.  One MFMA step consumes two chunk columns: lanes 0-31 give
// chunk 2s, lanes 32-63 chunk 2s+1 of rows (lane mod 32); the same assignment
// on both operands makes the contraction exact for any chunk order.
//   f16 / bf16: v_mfma_f32_32x32x16 (one MFMA per chunk pair)
//   f32:        v_mfma_f32_32x32x2  (four MFMAs per chunk pair)
// Accumulation is fp32; the epilogue applies alpha / beta / gamma in fp32 and
// rounds once to the output type.
#include "common.h"

namespace dion3 {

template <typename T> struct Mma;

template <> struct Mma<f16> {
  static constexpr int EPC = 8;
  __device__ static void run(floatx16& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                 __builtin_bit_cast(half8, b), acc, 0, 0, 0);
  }
};

template <> struct Mma<bf16_t> {
  static constexpr int EPC = 8;
  __device__ static void run(floatx16& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bfx8, a),
                                                  __builtin_bit_cast(bfx8, b), acc, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int EPC = 4;
  __device__ static void run(floatx16& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;          // bytes of K per LDS row per stage
constexpr int kChunks = kRowBytes / 16; // 8 chunks per row

struct KParams {
  int M, N, K;
  const void* A; long long lda, sA;
  const void* B; long long ldb, sB;
  const void* E; long long lde, sE;
  void* C; long long ldc, sC;
  float alpha, beta, gamma;
  int tiles_m, tiles_n, tiles_per_mat;
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

// Map a flat tile index to (ti, tj) with tj <= ti (lower triangle, diagonal included).
__device__ __forceinline__ void tri_index(int t, int& ti, int& tj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// Load one 16-byte chunk (EPC elements along K) of row `row` starting at
// element k, zero-filling anything outside [0, rows) x [0, K).
template <typename T, bool GUARD>
__device__ __forceinline__ uint4 load_chunk(const T* base, long long ld, int row, int rows, int k, int K) {
  constexpr int EPC = Mma<T>::EPC;
  if (!GUARD) return *(const uint4*)(base + (long long)row * ld + k);
  union { uint4 v; T e[EPC]; } u;
  u.v = make_uint4(0, 0, 0, 0);
  if (row < rows) {
    const T* p = base + (long long)row * ld;
#pragma unroll
    for (int e = 0; e < EPC; ++e)
      if (k + e < K) u.e[e] = p[k + e];
  }
  return u.v;
}

template <typename TO>
__device__ __forceinline__ void put(void* C, long long off, float v) {
  ((TO*)C)[off] = Store<TO>::from_f32(v);
}

// OP: GemmOp.  BT: B operand is an N-contiguous K x N matrix (X in Q X) that
// is transposed on its way into LDS.  SYM: lower-triangle tiles + mirror.
template <typename T, typename TO, int OP, bool GUARD, int BM>
__global__ __launch_bounds__(kThreads) void gemm_kernel(KParams p) {
  constexpr bool SYM = OP != OP_GEMM;
  constexpr bool BT = OP == OP_GEMM;
  constexpr int BN = BM;
  constexpr int EPC = Mma<T>::EPC;
  constexpr int BKE = kRowBytes / (int)sizeof(T);       // K elements per stage
  constexpr int WT = BM / 2;                             // wave tile edge
  constexpr int SUB = WT / 32;                           // 32x32 MFMA tiles per wave edge
  constexpr int A_LOADS = BM * kChunks / kThreads;       // chunks per thread per stage
  constexpr int B_LOADS = BN * kChunks / kThreads;

  __shared__ __attribute__((aligned(16))) char smem[2][2][BM * kRowBytes];

  // ---- tile scheduling (XCD-aware: consecutive tiles land on one XCD)
  const int G = gridDim.x;
  const int wg = blockIdx.x;
  const int per = G / 8;
  const int id = wg < per * 8 ? (wg % 8) * per + wg / 8 : wg;
  const int bat = id / p.tiles_per_mat;
  const int t = id % p.tiles_per_mat;
  int ti, tj;
  if (SYM) {
    tri_index(t, ti, tj);
  } else {
    ti = t % p.tiles_m;
    tj = t / p.tiles_m;
  }
  const int m0 = ti * BM, n0 = tj * BN;

  const T* A = (const T*)p.A + bat * p.sA;
  const T* B = (const T*)p.B + bat * p.sB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  floatx16 acc[SUB][SUB];
#pragma unroll
  for (int i = 0; i < SUB; ++i)
#pragma unroll
    for (int j = 0; j < SUB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[A_LOADS], rb[B_LOADS];

  auto load_stage = [&](int k0) {
#pragma unroll
    for (int s = 0; s < A_LOADS; ++s) {
      const int q = tid + kThreads * s;
      const int row = q / kChunks, c = q % kChunks;
      ra[s] = load_chunk<T, GUARD>(A, p.lda, m0 + row, p.M, k0 + c * EPC, p.K);
    }
    if (!BT) {
#pragma unroll
      for (int s = 0; s < B_LOADS; ++s) {
        const int q = tid + kThreads * s;
        const int row = q / kChunks, c = q % kChunks;
        rb[s] = load_chunk<T, GUARD>(B, p.ldb, n0 + row, p.N, k0 + c * EPC, p.K);
      }
    } else {
      // X is K x N row-major: a stage is BKE rows of BN elements, BN/EPC chunks per row
      constexpr int CPR = BN / EPC;
#pragma unroll
      for (int s = 0; s < B_LOADS; ++s) {
        const int q = tid + kThreads * s;
        const int kr = q / CPR, nc = q % CPR;
        rb[s] = load_chunk<T, GUARD>(B, p.ldb, k0 + kr, p.K, n0 + nc * EPC, p.N);
      }
    }
  };

  auto store_stage = [&](int buf) {
    char* sa = smem[buf][0];
    char* sb = smem[buf][1];
#pragma unroll
    for (int s = 0; s < A_LOADS; ++s) {
      const int q = tid + kThreads * s;
      *(uint4*)(sa + swz(q / kChunks, q % kChunks)) = ra[s];
    }
    if (!BT) {
#pragma unroll
      for (int s = 0; s < B_LOADS; ++s) {
        const int q = tid + kThreads * s;
        *(uint4*)(sb + swz(q / kChunks, q % kChunks)) = rb[s];
      }
    } else {
      constexpr int CPR = BN / EPC;
#pragma unroll
      for (int s = 0; s < B_LOADS; ++s) {
        const int q = tid + kThreads * s;
        const int kr = q / CPR, nc = q % CPR;
        union { uint4 v; T e[EPC]; } u;
        u.v = rb[s];
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const int n = nc * EPC + e;
          *(T*)(sb + swz(n, kr / EPC) + (kr % EPC) * (int)sizeof(T)) = u.e[e];
        }
      }
    }
  };

  const int KT = (p.K + BKE - 1) / BKE;
  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_stage((kt + 1) * BKE);
    const char* sa = smem[cur][0];
    const char* sb = smem[cur][1];
#pragma unroll
    for (int s = 0; s < kChunks / 2; ++s) {
      const int chunk = 2 * s + (lane >> 5);
      uint4 fa[SUB], fb[SUB];
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        const int row = wm * WT + i * 32 + (lane & 31);
        fa[i] = *(const uint4*)(sa + swz(row, chunk));
      }
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        const int row = wn * WT + j * 32 + (lane & 31);
        fb[j] = *(const uint4*)(sb + swz(row, chunk));
      }
#pragma unroll
      for (int i = 0; i < SUB; ++i)
#pragma unroll
        for (int j = 0; j < SUB; ++j) Mma<T>::run(acc[i][j], fa[i], fb[j]);
    }
    if (kt + 1 < KT) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  TO* C = (TO*)p.C + bat * p.sC;
  const TO* E = (const TO*)p.E + (p.E ? bat * p.sE : 0);
  const bool diag = SYM && ti == tj;
#pragma unroll
  for (int i = 0; i < SUB; ++i)
#pragma unroll
    for (int j = 0; j < SUB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gi = m0 + wm * WT + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int gj = n0 + wn * WT + j * 32 + (lane & 31);
        if (GUARD && (gi >= p.M || gj >= p.N)) continue;
        if (diag && gi < gj) continue;                  // upper half of a diagonal tile
        float v = p.alpha * acc[i][j][r];
        if (OP == OP_SYRK) {
          if (p.beta != 0.f) v += p.beta * Store<TO>::to_f32(E[(long long)gi * p.lde + gj]);
        } else if (OP == OP_SQ_ADD) {
          v += p.beta * Store<TO>::to_f32(E[(long long)gi * p.lde + gj]);
          if (gi == gj) v += p.gamma;
        }
        put<TO>(C, (long long)gi * p.ldc + gj, v);
        if (SYM && gi != gj) put<TO>(C, (long long)gj * p.ldc + gi, v);
      }
}

template <typename T, typename TO, int OP, int BM>
static int launch_typed(const GemmArgs& a, hipStream_t s) {
  constexpr int BKE = kRowBytes / (int)sizeof(T);
  constexpr int EPC = Mma<T>::EPC;
  KParams p;
  p.M = a.M; p.N = a.N; p.K = a.K;
  p.A = a.A; p.lda = a.lda; p.sA = a.sA;
  p.B = a.B; p.ldb = a.ldb; p.sB = a.sB;
  p.E = a.E; p.lde = a.lde; p.sE = a.sE;
  p.C = a.C; p.ldc = a.ldc; p.sC = a.sC;
  p.alpha = a.alpha; p.beta = a.beta; p.gamma = a.gamma;
  p.tiles_m = (a.M + BM - 1) / BM;
  p.tiles_n = (a.N + BM - 1) / BM;
  p.tiles_per_mat = OP == OP_GEMM ? p.tiles_m * p.tiles_n : p.tiles_m * (p.tiles_m + 1) / 2;
  const long long grid = (long long)p.tiles_per_mat * a.batch;
  if (grid <= 0 || grid > 0x7fffffffLL) return DION3_ERR_UNSUPPORTED;

  const bool bt = OP == OP_GEMM;
  bool fast = a.M % BM == 0 && a.N % BM == 0 && a.K % BKE == 0 &&
              a.lda % EPC == 0 && a.ldb % EPC == 0 && aligned16(a.A) && aligned16(a.B) &&
              (a.batch == 1 || (a.sA % EPC == 0 && a.sB % EPC == 0));
  (void)bt;
  static const char* names[4] = {"syrk", "sym_sq_add", "sym_mul", "gemm_qx"};
  TimedLaunch tl(names[OP], s);
  if (fast)
    hipLaunchKernelGGL((gemm_kernel<T, TO, OP, false, BM>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_kernel<T, TO, OP, true, BM>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return launch_status();
}

template <int OP>
static int dispatch(const GemmArgs& a, hipStream_t s) {
  constexpr int BM = 128;
  if (a.dtype == DION3_F16) {
    if (a.out_dtype == DION3_F16) return launch_typed<f16, f16, OP, BM>(a, s);
    if (a.out_dtype == DION3_F32 && OP == OP_GEMM) return launch_typed<f16, float, OP, BM>(a, s);
  } else if (a.dtype == DION3_BF16) {
    if (a.out_dtype == DION3_BF16) return launch_typed<bf16_t, bf16_t, OP, BM>(a, s);
  } else if (a.dtype == DION3_F32) {
    if (a.out_dtype == DION3_F32) return launch_typed<float, float, OP, BM>(a, s);
  }
  return DION3_ERR_INVALID_ARG;
}

int launch_gemm(const GemmArgs& a, hipStream_t s) {
  switch (a.op) {
    case OP_SYRK: return dispatch<OP_SYRK>(a, s);
    case OP_SQ_ADD: return dispatch<OP_SQ_ADD>(a, s);
    case OP_SYM_MUL: return dispatch<OP_SYM_MUL>(a, s);
    case OP_GEMM: return dispatch<OP_GEMM>(a, s);
  }
  return DION3_ERR_INVALID_ARG;
}

}  // namespace dion3
