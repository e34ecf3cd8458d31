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
// XOR-swizzled by the row so that the lanes of one LDS read phase reading a
// chunk column hit distinct banks.  One MFMA step consumes two chunk columns: lanes 0-31 give
// chunk 2s, lanes 32-63 chunk 2s+1 of rows (lane mod 32); the same assignment
// on both operands makes the contraction exact for any chunk order.
//   f16 / bf16: v_mfma_f32_32x32x16 (one MFMA per chunk pair)
//   f32:        v_mfma_f32_32x32x2  (four MFMAs per chunk pair)
// Accumulation is fp32; the epilogue applies alpha / beta / gamma in fp32 as
// fma(beta, e, alpha acc) + gamma and rounds that fp32 value to the output
// type, written out the same way in every kernel, so that a matrix's result
// does not depend on the tile size its batch gets.
#include <type_traits>

#include "common.h"

namespace dion3 {

template <typename T> struct Mma;

template <> struct Mma<f16> {
  static constexpr int EPC = 8;
  __device__ static void run(floatx16& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                 __builtin_bit_cast(half8, b), acc, 0, 0, 0);
  }
  // acc = a b (the accumulator input is zero)
  __device__ static void first(floatx16& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                 __builtin_bit_cast(half8, b), floatx16{}, 0, 0, 0);
  }
};

template <> struct Mma<bf16_t> {
  static constexpr int EPC = 8;
  __device__ static void run(floatx16& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bfx8, a),
                                                  __builtin_bit_cast(bfx8, b), acc, 0, 0, 0);
  }
  __device__ static void first(floatx16& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bfx8, a),
                                                  __builtin_bit_cast(bfx8, b), floatx16{}, 0, 0, 0);
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
#ifndef DION3_STAGES
#define DION3_STAGES 5
#endif
constexpr int kStages = DION3_STAGES;   // LDS stages of the large-tile kernel
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
  int ntiles;          // tiles over the batch
  int tiles_per_wg;    // large-tile kernel: tiles run back to back by one work-group
  int reverse;         // batch visited from its last matrix
  int same;            // symmetric kernels: B is A (same pointer, leading dimension and stride)
  // fused update (large-tile Q X with APPLY): see GemmArgs
  void* W; long long sW; int wlines; const int32_t* idx;
  float eta, u; int decay;
};

// LDS position of 16-byte chunk `chunk` of tile row `row`.  A 128-bit LDS read
// is served 16 lanes (256 bytes, all 64 banks) at a time; 16 lanes reading one
// chunk column of 16 consecutive rows must hit 16 distinct 16-byte slots.
// Rows alternate between the two 128-byte halves of a 256-byte line, and
// (row / 2) mod 8 permutes the chunk inside the half.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row >> 1) & 7)) << 4);
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

// The epilogue's fp32 value rounded to the output type.  The empty asm makes
// the fp32 value opaque, so the compiler cannot fuse the multiply-add before
// it and the rounding into one mixed-precision instruction (which rounds once,
// from the exact value): it would do so on some code paths and not on others,
// and the tile kernels would then disagree in the last bit.
template <typename TO>
__device__ __forceinline__ TO epi_round(float v) {
  asm("" : "+v"(v));
  return Store<TO>::from_f32(v);
}

template <typename TO>
__device__ __forceinline__ void put(void* C, long long off, float v) {
  ((TO*)C)[off] = epi_round<TO>(v);
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
  const int t = id % p.tiles_per_mat;
  const int bat = p.reverse ? p.ntiles / p.tiles_per_mat - 1 - id / p.tiles_per_mat : id / p.tiles_per_mat;
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
          if (p.beta != 0.f) v = __builtin_fmaf(p.beta, Store<TO>::to_f32(E[(long long)gi * p.lde + gj]), v);
        } else if (OP == OP_SQ_ADD) {
          v = __builtin_fmaf(p.beta, Store<TO>::to_f32(E[(long long)gi * p.lde + gj]), v);
          if (gi == gj) v += p.gamma;
        }
        put<TO>(C, (long long)gi * p.ldc + gj, v);
        if (SYM && gi != gj) put<TO>(C, (long long)gj * p.ldc + gi, v);
      }
}


// ---------------------------------------------------------------------------
// Large-tile kernel for fp16 / bf16: a 256 x 256 tile per work-group, 4 waves
// in 2 x 2, each wave owning a 128 x 128 block (4 x 4 MFMA 32x32x16 tiles), so
// every 16-byte fragment read from LDS feeds four MFMAs.  A stage holds 32 K
// elements of both operands (32 KB); NBUF stages rotate through LDS.
//
// Operands travel from global memory straight into LDS with buffer loads that
// write LDS directly (each lane's 16 bytes land at the wave's LDS base + 16 x
// lane), so no registers are spent on staging.  K-contiguous operands land as
// 64-byte rows with a row-dependent chunk swizzle; the N-contiguous X of Q X
// lands as 512-byte rows and its MFMA fragments come from transposing LDS
// reads (ds_read_b64_tr_b16), which hand each lane four consecutive K values
// of one column.  MFMA fragments are double-buffered across k-steps so LDS
// latency overlaps the MFMAs of the previous step.
//
// Q X runs several tiles per work-group: the stage sequence continues from one
// tile into the next, so the next tile's first stages are loaded while the
// current tile finishes, and the MFMA computes C^T blocks (operands swapped),
// which leaves four consecutive columns of one row in each lane; lane swaps
// across the half-waves and 16-lane rows form 16-byte row chunks, and an
// exchange between lanes L and L ^ 8 of two neighbouring blocks lets each
// store write 8 rows x 128 contiguous bytes; a tile is written with 32 stores
// per lane that stay in flight while the next tile computes.
// ---------------------------------------------------------------------------
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// Buffer resource (four scalar dwords) for raw loads of `bytes` bytes from
// `base`; the last dword is the gfx9 raw-buffer format word.
typedef int int4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int4v make_rsrc(const void* base, long long bytes) {
  const unsigned long long a = (unsigned long long)base;
  int4v r;
  r.x = __builtin_amdgcn_readfirstlane((int)(a & 0xffffffffu));
  r.y = __builtin_amdgcn_readfirstlane((int)(a >> 32) & 0xffff);    // stride 0
  r.z = __builtin_amdgcn_readfirstlane(bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
  r.w = 0x00020000;
  return r;
}

// One wave instruction: 64 lanes x 16 bytes from rsrc at voffset + soffset
// into LDS at byte address `lds` (wave-uniform) + 16 x lane.  Issued from
// inline assembly so that the compiler does not wait for it before unrelated
// LDS reads: the caller waits (vmcnt) before the barrier that publishes the
// stage.
__device__ __forceinline__ void lds_dma16(const int4v& rsrc, unsigned lds, int voffset, int soffset) {
  const int m0 = __builtin_amdgcn_readfirstlane((int)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m0), "v"(voffset), "s"(rsrc), "s"(soffset) : "memory", "m0");
}

// LDS position of 16-byte chunk `chunk` of row `row` of a K-contiguous operand
// stage (32 K elements = 64 bytes per row).  The 16 lanes of an LDS read phase
// read one chunk column of 16 consecutive rows: 4 rows share each 256-byte
// line and (row / 4) mod 4 permutes the chunk within its 64 bytes.
__device__ __forceinline__ int swz32(int row, int chunk) {
  return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4);
}

// N-contiguous stage (32 rows of 256 elements, 512 bytes): 16-byte chunk ch
// of row kr sits at slot nslot(kr, ch) = t(ch) xor 2 (kr mod 4), where t flips
// bit 3 of ch when bit 1 is set (an involution).  A transposing LDS read phase
// reads, per 32 lanes, four rows (kr mod 4 = 0..3) x four chunks (two pairs
// 2 apart, from the two 16-lane halves): the xor 2 (kr mod 4) spreads one
// half over 8 slots of a 128-byte bank cycle, and t moves the other half to
// the other 8 slots of 256 bytes, so neither 32 nor 64 four-byte banks see a
// conflict (measured on MI355X: the plain xor 2 (kr mod 4) made these reads
// 2-way conflicted).
__device__ __forceinline__ int nslot(int kr, int ch) {
  return (ch ^ (((ch >> 1) & 1) << 3)) ^ (2 * (kr & 3));
}
// the chunk that belongs in slot s of row kr (the inverse of nslot)
__device__ __forceinline__ int nchunk(int kr, int s) {
  const int u = s ^ (2 * (kr & 3));
  return u ^ (((u >> 1) & 1) << 3);
}
// Byte offset of element column n (a multiple of 4) of row kr.
__device__ __forceinline__ int swzn(int kr, int n) {
  return kr * 512 + (nslot(kr, n >> 3) << 4) + ((n & 4) << 1);
}

// Wait until at most n vector memory operations of this wave are outstanding
// (0 <= n <= 63, the counter's range; larger n waits as for 63).  The counter
// retires loads and stores in issue order.
#define DION3_VM_CASE(k) \
  case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
#define DION3_VM_CASE8(k) DION3_VM_CASE(k) DION3_VM_CASE(k + 1) DION3_VM_CASE(k + 2) DION3_VM_CASE(k + 3) \
  DION3_VM_CASE(k + 4) DION3_VM_CASE(k + 5) DION3_VM_CASE(k + 6) DION3_VM_CASE(k + 7)
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    DION3_VM_CASE8(0) DION3_VM_CASE8(8) DION3_VM_CASE8(16) DION3_VM_CASE8(24)
    DION3_VM_CASE8(32) DION3_VM_CASE8(40) DION3_VM_CASE8(48) DION3_VM_CASE8(56)
    default:
      if (n > 63) asm volatile("s_waitcnt vmcnt(63)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      break;
  }
}
#undef DION3_VM_CASE8
#undef DION3_VM_CASE

// End-of-stage barrier of the large-tile kernel.  The stage's DMA has been
// waited for (vmcnt) before it; LDS reads need no wait here: every read of the
// buffer the next DMA overwrites was consumed by an MFMA of this stage, and
// the reads still in flight target the next stage's buffer.  (__syncthreads
// would add a wait for all LDS reads, including those prefetched fragments.)
// The memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_barrier" ::: "memory");
}

typedef short short4v __attribute__((ext_vector_type(4)));

// Read one accumulator out of its AGPR where it is used (an inline read keeps
// the register allocator from copying every accumulator to VGPRs at once).
__device__ __forceinline__ float acc_read(float v) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(v));
  return r;
}

// Row chunks of a 32 x 32 block for 64-byte stores.  On entry lane L holds
// the 16-byte chunks w0 (columns 8 (L/32) .. + 7) and w1 (columns 16 + 8 (L/32)
// .. + 7) of block row L mod 32.  v_permlane16_swap exchanges the odd 16-lane
// rows of its first operand with the even 16-lane rows of its second, which
// leaves a = the chunk of block row L mod 16 and b = that of row 16 + L mod 16,
// both at column 16 ((L / 16) mod 2) + 8 (L / 32): one store of a (or of b)
// across the wave writes 16 rows x 64 contiguous bytes.
__device__ __forceinline__ void rows64(const uint4& w0, const uint4& w1, uint4& a, uint4& b) {
  const auto x = __builtin_amdgcn_permlane16_swap(w0.x, w1.x, false, false);
  const auto y = __builtin_amdgcn_permlane16_swap(w0.y, w1.y, false, false);
  const auto z = __builtin_amdgcn_permlane16_swap(w0.z, w1.z, false, false);
  const auto w = __builtin_amdgcn_permlane16_swap(w0.w, w1.w, false, false);
  a = make_uint4(x[0], y[0], z[0], w[0]);
  b = make_uint4(x[1], y[1], z[1], w[1]);
}

__device__ __forceinline__ uint4 sel4(bool c, const uint4 u, const uint4 v) {
  return make_uint4(c ? u.x : v.x, c ? u.y : v.y, c ? u.z : v.z, c ? u.w : v.w);
}

// Exchange between lanes L and L ^ 8 (DPP row rotation by 8 within 16 lanes).
__device__ __forceinline__ uint4 xchg8(const uint4& v) {
  return make_uint4((unsigned)__builtin_amdgcn_mov_dpp((int)v.x, 0x128, 0xf, 0xf, false),
                    (unsigned)__builtin_amdgcn_mov_dpp((int)v.y, 0x128, 0xf, 0xf, false),
                    (unsigned)__builtin_amdgcn_mov_dpp((int)v.z, 0x128, 0xf, 0xf, false),
                    (unsigned)__builtin_amdgcn_mov_dpp((int)v.w, 0x128, 0xf, 0xf, false));
}

struct TileAddr {
  int4v ra, rb;      // buffer resources based at the tile's first A row / B row or column
  int m0, n0, bat, ti, tj;
  int bo;            // byte offset of the B fragments in a stage buffer
};

constexpr int kEpiStores = 32;   // 16-byte stores per wave in a Q X tile epilogue

// 16-byte accesses of W rows in the fused update (each byte touched once)
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u x = __builtin_nontemporal_load((const v4u*)p);
  return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void st_nt16(void* p, const uint4& v) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, (v4u*)p);
}

// update_w on 8 consecutive entries: W chunk w (bf16) with the rounded
// results o (8 values of type TO) of the same columns
// (update_w's arithmetic; the two results of a pair rounded by one
// instruction, bit-identical to rounding each)
template <typename TO>
__device__ __forceinline__ uint4 update8(const uint4& w, const uint4& o, float eta, float u, bool decay) {
  union { uint4 v; bf16_t e[8]; } wu;
  union { uint4 v; TO e[8]; } ou;
  union { uint4 v; uint32_t d[4]; } r;
  wu.v = w;
  ou.v = o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float a0 = bf16_to_f32(wu.e[2 * q]), a1 = bf16_to_f32(wu.e[2 * q + 1]);
    if (decay) { a0 = u * a0; a1 = u * a1; }
    r.d[q] = f32x2_to_bf16x2(__builtin_fmaf(-eta, Store<TO>::to_f32(ou.e[2 * q]), a0),
                             __builtin_fmaf(-eta, Store<TO>::to_f32(ou.e[2 * q + 1]), a1));
  }
  return r.v;
}

typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v* lds_s4_ptr;

// 16-byte LDS read at byte address `addr`
__device__ __forceinline__ uint4 lds_read16(unsigned addr) {
  const u32x4v v = *(const __attribute__((address_space(3))) u32x4v*)(uintptr_t)addr;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Large-tile kernel (fp16 / bf16, whole tiles only).  Global stage g (stage g
// mod KT of the work-group's tile g / KT) lives in LDS buffer g mod NBUF.  Its
// loads are issued right after the barrier that ends stage g - NBUF (the last
// use of that buffer) and must have landed by the barrier that ends stage
// g - 2; the first k-step's fragments of stage g are then read during stage
// g - 1, so a wave leaves every barrier with its next MFMA operands in
// registers.  Each wave issues 8 one-kilobyte DMA instructions per stage.
//
// APPLY (Q X only): the epilogue does not store the tile; each 16-byte chunk
// of it (rounded to TO exactly as stored) updates the same columns of W row
// idx[b][r] instead, the chunks of W loaded together at the start of the
// epilogue.  Every store instruction is still issued (a row whose index is
// out of range stores its chunk to C), so the count of stores in flight that
// the next tile's waits allow for is the same.
template <typename T, typename TO, int OP, int NBUF, bool APPLY = false>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm256_kernel(KParams p) {
  static_assert(!APPLY || (OP == OP_GEMM && sizeof(TO) == 2), "the update is fused into Q X only");
  constexpr bool SYM = OP != OP_GEMM;
  constexpr bool BT = OP == OP_GEMM;
  constexpr bool SWAP = true;                       // MFMA produces C^T blocks
  constexpr bool MULTI = sizeof(TO) == 2;           // several tiles per work-group
  constexpr int BM = 256, BN = 256;
  constexpr int BK = 32;                      // K elements per stage
  constexpr int WT = 128;                     // wave tile edge
  constexpr int SUB = WT / 32;                // 4 x 4 MFMA tiles per wave
  constexpr int STAGE = 32768;                // bytes per stage (both operands)

  __shared__ __attribute__((aligned(1024))) char smem[NBUF * STAGE];
  const unsigned lds0 = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)smem;

  // XCD-aware order: consecutive ids run on one XCD at the same time
  const int G = gridDim.x;
  const int wg = blockIdx.x;
  const int per = G / 8;
  const int id = wg < per * 8 ? (wg % 8) * per + wg / 8 : wg;
  // this work-group's tiles: id, id + G, ... (fewer at the end of the range)
  const int nt = MULTI ? min(p.tiles_per_wg, (p.ntiles - id + G - 1) / G) : 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar LDS offsets
  const int wm = wave >> 1, wn = wave & 1;

  // ---- DMA addressing (per-lane offsets from the tile's buffer base).
  // K-contiguous operand: wave instruction q (0..3) covers tile rows
  // 64 q + 16 wave + [0, 16); lane L fetches row 64 q + 16 wave + L/4 and the
  // chunk whose swizzled position is L mod 4.  N-contiguous B (Q X):
  // instruction q covers stage rows 8 q + 2 wave + {0, 1}; lane L fetches row
  // 8 q + 2 wave + L/32, the chunk whose swizzled position is L mod 32.
  const int va = ((16 * wave + (lane >> 2)) * (int)p.lda + (((lane & 3) ^ (lane >> 4)) << 3)) * 2;
  const int ka = 64 * (int)p.lda * 2;                 // +64 rows per instruction
  int vb, kb;
  if (!BT) {
    vb = ((16 * wave + (lane >> 2)) * (int)p.ldb + (((lane & 3) ^ (lane >> 4)) << 3)) * 2;
    kb = 64 * (int)p.ldb * 2;
  } else {
    const int kr = 2 * wave + (lane >> 5);
    vb = (kr * (int)p.ldb + (nchunk(kr, lane & 31) << 3)) * 2;
    kb = 8 * (int)p.ldb * 2;                          // +8 rows per instruction
  }
  auto tile_addr = [&](int L, TileAddr& a) {
    int bat = L / p.tiles_per_mat;
    const int t = L - bat * p.tiles_per_mat;
    if (p.reverse) bat = p.ntiles / p.tiles_per_mat - 1 - bat;
    int ti, tj;
    if (SYM) {
      tri_index(t, ti, tj);
    } else {
      ti = t % p.tiles_m;
      tj = t / p.tiles_m;
    }
    // the tile coordinates are uniform: keep them (and the buffer resources
    // derived from them) in scalar registers
    a.ti = __builtin_amdgcn_readfirstlane(ti);
    a.tj = __builtin_amdgcn_readfirstlane(tj);
    a.bat = __builtin_amdgcn_readfirstlane(bat);
    a.m0 = a.ti * BM;
    a.n0 = a.tj * BN;
    const T* A = (const T*)p.A + a.bat * p.sA + (long long)a.m0 * p.lda;
    const T* B = (const T*)p.B + a.bat * p.sB + (BT ? (long long)a.n0 : (long long)a.n0 * p.ldb);
    // a diagonal tile of a product whose B is A needs one operand panel:
    // its B fragments are read from the A half of each stage, and its B
    // loads, still issued so that every stage counts the same loads, go to
    // a resource of zero bytes (out of range: no memory access)
    // (the wave of the quadrant above the diagonal, whose results are never
    // stored, reads the B half instead: the out-of-range loads leave zeros
    // there, and MFMAs on zeros draw less power)
    const bool one_panel = SYM && p.same && a.ti == a.tj;
    a.bo = one_panel && wm >= wn ? 0 : 16384;
    a.ra = make_rsrc(A, (long long)(p.M - a.m0) * p.lda * 2);
    a.rb = make_rsrc(B, one_panel ? 0LL
                        : BT ? (long long)p.K * p.ldb * 2 - (long long)a.n0 * 2
                             : (long long)(p.N - a.n0) * p.ldb * 2);
  };

  // one DMA instruction x (0..3: operand A, 4..7: operand B) of the tile's
  // stage ls into LDS buffer b
  auto dma = [&](const int4v& ra, const int4v& rb, int ls, int b, int x) {
    const unsigned buf = lds0 + (unsigned)(b * STAGE);
    const int k0 = ls * BK;
    const int q = x & 3;
    if (x < 4) {
      lds_dma16(ra, buf + (64 * q + 16 * wave) * 64, va, k0 * 2 + q * ka);
    } else if (!BT) {
      lds_dma16(rb, buf + 16384 + (64 * q + 16 * wave) * 64, vb, k0 * 2 + q * kb);
    } else {
      lds_dma16(rb, buf + 16384 + (8 * q + 2 * wave) * 512, vb, k0 * (int)p.ldb * 2 + q * kb);
    }
  };

  // fragments of one k-step (16 K elements) of the stage in LDS buffer b:
  // A rows wm*128 + 32 i + lane%32; B either likewise (K-contiguous) or
  // through transposing reads (Q X)
  auto read_a = [&](uint4& f, int b, int st, int i) {
    const unsigned buf = lds0 + (unsigned)(b * STAGE);
    f = lds_read16(buf + swz32(wm * WT + i * 32 + (lane & 31), 2 * st + (lane >> 5)));
  };
  auto read_b = [&](uint4& f, int b, int st, int j, int bo) {
    const unsigned buf = lds0 + (unsigned)(b * STAGE) + (unsigned)bo;
    if (!BT) {
      f = lds_read16(buf + swz32(wn * WT + j * 32 + (lane & 31), 2 * st + (lane >> 5)));
    } else {
      // lane = 16 g + 4 q + t addresses row 16 st + 8 (g/2) + 4 h + q and
      // columns 16 (g mod 2) + 4 t .. +3 of the fragment's 32; the transposing
      // read hands each lane its column's four consecutive K values
      const int gg = lane >> 4, q = (lane >> 2) & 3, tt = lane & 3;
      const int n = wn * WT + j * 32 + 16 * (gg & 1) + 4 * tt;
      const int kr0 = 16 * st + 8 * (gg >> 1) + q;
      const short4v h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(uintptr_t)(buf + swzn(kr0, n)));
      const short4v h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(uintptr_t)(buf + swzn(kr0 + 4, n)));
      f = make_uint4(__builtin_bit_cast(uint2, h0).x, __builtin_bit_cast(uint2, h0).y,
                     __builtin_bit_cast(uint2, h1).x, __builtin_bit_cast(uint2, h1).y);
    }
  };

  // accumulators: the first k-step of every tile overwrites them (MFMA with a
  // zero accumulator input), so they are dead between a tile's epilogue and
  // the next tile
  floatx16 acc[SUB][SUB];

  // APPLY: the W row index of each output row this lane stores (rows
  // m0 + 128 wm + (lane mod 8) + 32 i + 16 hh + 8 e of the tile), for the
  // current tile and, loaded during its epilogue, the next one
  int wr[SUB][2][2], wr_next[SUB][2][2];
  auto load_rows = [&](const TileAddr& a, int (&dst)[SUB][2][2]) {
    const int32_t* ib = p.idx + (long long)a.bat * p.M + a.m0 + wm * WT + (lane & 7);
    static_for<SUB>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      static_for<2>([&](auto hc) {
        constexpr int hh = decltype(hc)::value;
        static_for<2>([&](auto ec) {
          constexpr int e = decltype(ec)::value;
          dst[i][hh][e] = ib[32 * i + 16 * hh + 8 * e];
        });
      });
    });
  };

  // Q X epilogue: block (i, j) of the wave holds C[row lane%32][8 g + 4 (lane/32)
  // + 0..3] in acc[i][j][4 g .. 4 g + 3]; a lane swap across the half-waves gives
  // lane L < 32 columns 16 h .. +7 and lane L + 32 columns 16 h + 8 .. +15
  auto epilogue_swap = [&](const TileAddr& a, const TileAddr& an, bool more) {
    if constexpr (SWAP) {
      TO* C = (TO*)p.C + a.bat * p.sC;
      const int lc = lane & 31, lh = lane >> 5;
      TO* rowp = C + (long long)(a.m0 + wm * WT + lc) * p.ldc + (a.n0 + wn * WT);
      // 16-bit output, blocks (i, 2 jp) and (i, 2 jp + 1) together: after
      // rows64 lane L holds, for both blocks, the chunk at column
      // 16 ((L / 16) mod 2) + 8 (L / 32) of block row r = L mod 16 (+ 16); lanes
      // L and L ^ 8 (rows r and r ^ 8) exchange one chunk each (DPP rotation by
      // 8 within 16 lanes), so that one store writes 8 rows x 128 contiguous
      // bytes (64 columns)
      const int hi8 = (lc >> 3) & 1;
      TO* rowo = C + (long long)(a.m0 + wm * WT + (lc & 7)) * p.ldc + (a.n0 + wn * WT) + 32 * hi8 +
                 16 * ((lc >> 4) & 1) + 8 * lh;
      // APPLY: the next tile's row indices, then the W chunks these stores
      // update (row wr[i][hh][e], columns cw + 64 jj .. + 7), all loaded
      // before the first is needed (the waits for the chunks, in issue order,
      // also complete the indices)
      bf16_t* Wb = nullptr;
      int cw = 0;
      uint4 wv[SUB][2][2][2];
      if constexpr (APPLY) {
        if (more) load_rows(an, wr_next);
        Wb = (bf16_t*)p.W + a.bat * p.sW;
        cw = a.n0 + wn * WT + 32 * hi8 + 16 * ((lc >> 4) & 1) + 8 * lh;
        static_for<SUB>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          static_for<2>([&](auto hc) {
            constexpr int hh = decltype(hc)::value;
            static_for<2>([&](auto ec) {
              constexpr int e = decltype(ec)::value;
              // an out-of-range row loads row 0 (unused): every load is issued,
              // so the waits for them can be counted
              const int r = (unsigned)wr[i][hh][e] < (unsigned)p.wlines ? wr[i][hh][e] : 0;
              static_for<2>([&](auto jc) {
                constexpr int jj = decltype(jc)::value;
                wv[i][hh][e][jj] = ld_nt16(Wb + (long long)r * p.N + cw + 64 * jj);
              });
            });
          });
        });
        __builtin_amdgcn_sched_barrier(0);
      }
      // one block's results as two 64-byte row chunks per lane (rows64)
      auto chunks = [&](auto ic, auto jc, uint4& ra, uint4& rb) {
        if constexpr (sizeof(TO) == 2) {
        constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
        uint32_t d[4][2];
        static_for<4>([&](auto gc) {
          constexpr int g = decltype(gc)::value;
          static_for<2>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            const TO lo = epi_round<TO>(p.alpha * acc_read(acc[i][j][4 * g + 2 * h]));
            const TO hi = epi_round<TO>(p.alpha * acc_read(acc[i][j][4 * g + 2 * h + 1]));
            d[g][h] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          });
        });
        uint4 w[2];
        static_for<2>([&](auto pc) {
          constexpr int pr = decltype(pc)::value;
          const auto s0 = __builtin_amdgcn_permlane32_swap(d[2 * pr][0], d[2 * pr + 1][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(d[2 * pr][1], d[2 * pr + 1][1], false, false);
          w[pr] = make_uint4(s0[0], s1[0], s0[1], s1[1]);
        });
        rows64(w[0], w[1], ra, rb);
        }
      };
      static_for<SUB>([&](auto ic) {
        static_for<SUB>([&](auto jc) {
          constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
          // one block (pair) at a time: keeps the scheduler from moving every
          // accumulator into vector registers at once
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (sizeof(TO) == 2) {
            if constexpr (j % 2 == 0) {
              uint4 ra0, rb0, ra1, rb1;
              chunks(ic, jc, ra0, rb0);
              chunks(ic, std::integral_constant<int, j + 1>{}, ra1, rb1);
              static_for<2>([&](auto hc) {
                constexpr int hh = decltype(hc)::value;      // block rows 0-15 or 16-31
                const uint4 x0 = hh ? rb0 : ra0;              // block j, row r (+ 16)
                const uint4 x1 = hh ? rb1 : ra1;              // block j + 1, row r (+ 16)
                const uint4 recv = xchg8(sel4(hi8, x0, x1));
                TO* q = rowo + (long long)(32 * i + 16 * hh) * p.ldc + 32 * j;
                const uint4 c0 = sel4(hi8, recv, x0);             // row r mod 8 (+ 16)
                const uint4 c1 = sel4(hi8, x1, recv);             // row 8 + r mod 8 (+ 16)
                if constexpr (APPLY) {
                  constexpr int jj = j / 2;
                  const int r0 = wr[i][hh][0], r1 = wr[i][hh][1];
                  const bool ok0 = (unsigned)r0 < (unsigned)p.wlines, ok1 = (unsigned)r1 < (unsigned)p.wlines;
                  void* d0 = ok0 ? (void*)(Wb + (long long)r0 * p.N + cw + 64 * jj) : (void*)q;
                  void* d1 = ok1 ? (void*)(Wb + (long long)r1 * p.N + cw + 64 * jj) : (void*)(q + 8 * p.ldc);
                  st_nt16(d0, ok0 ? update8<TO>(wv[i][hh][0][jj], c0, p.eta, p.u, p.decay != 0) : c0);
                  st_nt16(d1, ok1 ? update8<TO>(wv[i][hh][1][jj], c1, p.eta, p.u, p.decay != 0) : c1);
                } else {
                  *(uint4*)q = c0;
                  *(uint4*)(q + 8 * p.ldc) = c1;
                }
              });
            }
          } else {
            TO* dst = rowp + (long long)(32 * i) * p.ldc + 32 * j;
            static_for<4>([&](auto gc) {
              constexpr int g = decltype(gc)::value;
              *(float4*)(dst + 8 * g + 4 * lh) =
                  make_float4(p.alpha * acc_read(acc[i][j][4 * g]), p.alpha * acc_read(acc[i][j][4 * g + 1]),
                              p.alpha * acc_read(acc[i][j][4 * g + 2]), p.alpha * acc_read(acc[i][j][4 * g + 3]));
            });
          }
        });
      });
    }
  };

  const bool use_e = OP == OP_SQ_ADD || (OP == OP_SYRK && p.beta != 0.f);

  // Symmetric epilogue (several tiles per work-group, no LDS).  Block (i, j)
  // of the wave holds C[r][c] for r = lane%32 and c = 8 g + 4 (lane/32) + q in
  // acc[i][j][4 g + q] (the Q X layout).  Direct part: 16-byte chunks of rows
  // r mod 16 and 16 + r mod 16 (rows64); on full quadrants of the symmetric
  // product and A^2 + B, blocks (i, j) and (i, j + 1) are stored together as in
  // Q X (8 rows x 128 bytes per store).  Mirror part: in each group of 8 lanes (rows 8 o .. 8 o + 7
  // of the block), a butterfly transpose of the 8 packed dwords over lane
  // distances 4, 2, 1 leaves lane t = lane%8 the 8 rows of columns
  // c0 = 8 (t/2) + 4 (lane/32) + 2 (t mod 2) and c0 + 1, which are 16-byte
  // chunks of rows c0 and c0 + 1 of the transposed position.  Diagonal tiles:
  // the wave above the diagonal writes nothing (its quadrant is the mirror of
  // the one below), blocks above the diagonal of the two diagonal quadrants
  // likewise, and on a diagonal block the direct chunk keeps columns <= row
  // and the mirror chunk rows > column, so every entry is written once, from
  // the value computed at or below the diagonal; on full quadrants of those two
  // kernels the mirror chunks of blocks (i, j) and (i + 1, j) are stored
  // together after lanes t and t ^ 1 exchange one chunk (8 transposed rows x
  // 128 bytes per store).  The epilogue operand is read at the direct
  // position: by X X^T with beta all up front, by A^2 + B per block group one
  // group ahead.  Returns the number of stores every lane issues (a lower
  // bound of the wave's count).
  auto epilogue_sym = [&](const TileAddr& a) -> int {
    int nst = 0;
    if constexpr (SYM) {
      const bool diag_tile = a.ti == a.tj;
      if (diag_tile && wm < wn) return 0;
      const bool dq = diag_tile && wm == wn;
      TO* C = (TO*)p.C + a.bat * p.sC;
      const TO* E = (const TO*)p.E + (p.E ? a.bat * p.sE : 0);
      const int lc = lane & 31, lh = lane >> 5;
      const int o = lc >> 3, t = lc & 7;
      const long long rb0 = a.m0 + wm * WT;       // first C row of the quadrant
      const long long cb0 = a.n0 + wn * WT;       // first C column of the quadrant
      // the epilogue operand: X X^T with beta != 0 loads all of it up front;
      // A^2 + B loads it per block group, one group ahead (fewer registers)
      constexpr bool EGROUP = OP == OP_SQ_ADD;
      uint2 epk[EGROUP ? 1 : SUB][EGROUP ? 1 : SUB][4];
      if (!EGROUP && use_e) {
        static_for<SUB>([&](auto ic) {
          static_for<SUB>([&](auto jc) {
            constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
            if (dq && i < j) return;
            if constexpr (!EGROUP) {
              const TO* er = E + (rb0 + 32 * i + lc) * p.lde + cb0 + 32 * j + 4 * lh;
              static_for<4>([&](auto gc) {
                constexpr int g = decltype(gc)::value;
                epk[i][j][g] = *(const uint2*)(er + 8 * g);
              });
            }
          });
        });
        wait_vm(0);
      }
      // packed results of block (i, j): dword 2 g + h holds columns 8 g + 4 (lane/32) + 2 h, + 1
      // ev: the block's epilogue operand words (read only when use_e)
      auto pack = [&](auto ic, auto jc, bool dblk, uint32_t (&d)[8], const uint2 (&ev)[4]) {
        constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
        static_for<4>([&](auto gc) {
          constexpr int g = decltype(gc)::value;
          static_for<2>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            float v0 = p.alpha * acc_read(acc[i][j][4 * g + 2 * h]);
            float v1 = p.alpha * acc_read(acc[i][j][4 * g + 2 * h + 1]);
            if (use_e) {
              const uint32_t ew = h ? ev[g].y : ev[g].x;
              v0 = __builtin_fmaf(p.beta, Store<TO>::to_f32(__builtin_bit_cast(TO, (uint16_t)(ew & 0xffffu))), v0);
              v1 = __builtin_fmaf(p.beta, Store<TO>::to_f32(__builtin_bit_cast(TO, (uint16_t)(ew >> 16))), v1);
            }
            if (OP == OP_SQ_ADD && dblk) {
              if (8 * g + 4 * lh + 2 * h == lc) v0 += p.gamma;
              if (8 * g + 4 * lh + 2 * h + 1 == lc) v1 += p.gamma;
            }
            d[2 * g + h] = (uint32_t)__builtin_bit_cast(uint16_t, epi_round<TO>(v0)) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, epi_round<TO>(v1)) << 16);
          });
        });
      };
      auto load_e = [&](int i, int j, uint2 (&ev)[4]) {
        const TO* er = E + (rb0 + 32 * i + lc) * p.lde + cb0 + 32 * j + 4 * lh;
#pragma unroll
        for (int g = 0; g < 4; ++g) ev[g] = *(const uint2*)(er + 8 * g);
      };
      // after the half-wave swap lane L holds columns 16 pr + 8 (L/32) .. + 7 of
      // row L mod 32 (pr = 0, 1); rows64 regroups them into 64-byte row chunks
      // of rows L mod 16 (wr[0]) and 16 + L mod 16 (wr[1])
      auto direct_chunks = [&](const uint32_t (&d)[8], uint4 (&wr)[2]) {
        uint4 wpr[2];
        static_for<2>([&](auto pc) {
          constexpr int pr = decltype(pc)::value;
          const auto s0 = __builtin_amdgcn_permlane32_swap(d[4 * pr], d[4 * pr + 2], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(d[4 * pr + 1], d[4 * pr + 3], false, false);
          wpr[pr] = make_uint4(s0[0], s1[0], s0[1], s1[1]);
        });
        rows64(wpr[0], wpr[1], wr[0], wr[1]);
      };
      // mirror: transpose the 8 dwords across the 8 lanes of the group (lane t
      // = lane mod 8 of group o = (lane mod 32) / 8), which leaves 16-byte
      // chunks of rows c0 (ma) and c0 + 1 (mb) of the transposed position,
      // c0 = 8 (t/2) + 4 (lane/32) + 2 (t mod 2), columns 8 o .. + 7 of the block
      auto mirror_chunks = [&](uint32_t (&d)[8], uint4& ma, uint4& mb) {
        static_for<3>([&](auto sc) {
          constexpr int s = 4 >> decltype(sc)::value;
          const bool up = (t & s) != 0;
          static_for<8>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            if constexpr ((k & s) == 0) {
              constexpr int kk = k | s;
              const uint32_t send = up ? d[k] : d[kk];
              const uint32_t recv =
                  (uint32_t)__builtin_amdgcn_ds_swizzle((int)send, (s << 10) | 0x1f);
              if (up) d[k] = recv;
              else d[kk] = recv;
            }
          });
        });
        // dword k now holds row 8 o + k, columns c0 (low half) and c0 + 1
        ma = make_uint4((d[0] & 0xffffu) | (d[1] << 16), (d[2] & 0xffffu) | (d[3] << 16),
                        (d[4] & 0xffffu) | (d[5] << 16), (d[6] & 0xffffu) | (d[7] << 16));
        mb = make_uint4((d[0] >> 16) | (d[1] & 0xffff0000u), (d[2] >> 16) | (d[3] & 0xffff0000u),
                        (d[4] >> 16) | (d[5] & 0xffff0000u), (d[6] >> 16) | (d[7] & 0xffff0000u));
      };
      const int c0 = 8 * (t >> 1) + 4 * lh + 2 * (t & 1);
      auto mirror = [&](auto ic, auto jc, bool dblk, uint32_t (&d)[8]) {
        constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
        uint4 ma, mb;
        mirror_chunks(d, ma, mb);
        TO* mrow = C + (cb0 + 32 * j + c0) * p.ldc + rb0 + 32 * i + 8 * o;
        static_for<2>([&](auto bc) {
          constexpr int b = decltype(bc)::value;
          const uint4& w = b ? mb : ma;
          const int y = c0 + b;                 // block column = transposed row
          TO* dst = mrow + b * p.ldc;
          if (!dblk || 8 * o > y) {
            *(uint4*)dst = w;
          } else if (8 * o + 7 > y) {
            union { uint4 v; TO e[8]; } u;
            u.v = w;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (8 * o + e > y) dst[e] = u.e[e];
          }
        });
      };
      // (the symmetric product only: with the A^2 + B and X X^T epilogues the
      // pairing raised register use and slowed their main loop)
      if ((OP == OP_SYM_MUL || OP == OP_SQ_ADD) && !dq) {
        // a full quadrant: blocks (i, j) and (i, j + 1) stored together, lanes L
        // and L ^ 8 exchanging one chunk each (DPP rotation by 8 within 16
        // lanes), so that a direct store writes 8 rows x 128 contiguous bytes
        const int hi8 = (lc >> 3) & 1;
        TO* rowo = C + (rb0 + (lc & 7)) * p.ldc + cb0 + 32 * hi8 + 16 * ((lc >> 4) & 1) + 8 * lh;
        // mirror stores of blocks (i, j) and (i + 1, j) together: lanes t and
        // t ^ 1 (rows c0 and c0 + 2 of the transposed position) exchange one
        // chunk each (DPP quad permutation [1, 0, 3, 2]), so that one store
        // writes 8 transposed rows x 128 contiguous bytes
        const int t1 = t & 1;
        TO* mrow2 = C + (cb0 + c0 - 2 * t1) * p.ldc + rb0 + 32 * t1 + 8 * o;
        auto swap1 = [](const uint4& v) {
          return make_uint4((unsigned)__builtin_amdgcn_mov_dpp((int)v.x, 0xB1, 0xf, 0xf, false),
                            (unsigned)__builtin_amdgcn_mov_dpp((int)v.y, 0xB1, 0xf, 0xf, false),
                            (unsigned)__builtin_amdgcn_mov_dpp((int)v.z, 0xB1, 0xf, 0xf, false),
                            (unsigned)__builtin_amdgcn_mov_dpp((int)v.w, 0xB1, 0xf, 0xf, false));
        };
        // A^2 + B: the epilogue operand of group q is loaded during group q - 1
        uint2 eg[2][2][2][4];
        auto load_group = [&](int i, int j, uint2 (&e)[2][2][4]) {
          load_e(i, j, e[0][0]); load_e(i, j + 1, e[0][1]);
          load_e(i + 1, j, e[1][0]); load_e(i + 1, j + 1, e[1][1]);
        };
        if (OP == OP_SQ_ADD) load_group(0, 0, eg[0]);
        static_for<SUB / 2>([&](auto ipc) {
          static_for<SUB / 2>([&](auto jpc) {
            constexpr int i = 2 * decltype(ipc)::value, j = 2 * decltype(jpc)::value;
            constexpr int q = (i / 2) * (SUB / 2) + j / 2, qb = q & 1;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (OP == OP_SQ_ADD && q + 1 < (SUB / 2) * (SUB / 2)) {
              constexpr int qn = q + 1;
              load_group(2 * (qn / (SUB / 2)), 2 * (qn % (SUB / 2)), eg[qb ^ 1]);
            }
            uint32_t d[2][2][8];                       // blocks (i + a, j + b)
            static_for<2>([&](auto ac) {
              static_for<2>([&](auto bc) {
                constexpr int a2 = decltype(ac)::value, b2 = decltype(bc)::value;
                pack(std::integral_constant<int, i + a2>{}, std::integral_constant<int, j + b2>{}, false, d[a2][b2],
                     eg[qb][a2][b2]);
              });
            });
            // direct: blocks (i + a, j) and (i + a, j + 1)
            static_for<2>([&](auto ac) {
              constexpr int a2 = decltype(ac)::value;
              uint4 w0[2], w1[2];
              direct_chunks(d[a2][0], w0);
              direct_chunks(d[a2][1], w1);
              static_for<2>([&](auto hc) {
                constexpr int hh = decltype(hc)::value;       // block rows 0-15 or 16-31
                const uint4 recv = xchg8(sel4(hi8, w0[hh], w1[hh]));
                TO* q = rowo + (32 * (i + a2) + 16 * hh) * p.ldc + 32 * j;
                *(uint4*)q = sel4(hi8, recv, w0[hh]);                 // row r mod 8 (+ 16)
                *(uint4*)(q + 8 * p.ldc) = sel4(hi8, w1[hh], recv);   // row 8 + r mod 8 (+ 16)
              });
            });
            // mirror: blocks (i, j + b) and (i + 1, j + b)
            static_for<2>([&](auto bc) {
              constexpr int b2 = decltype(bc)::value;
              uint4 m0a, m0b, m1a, m1b;                  // block rows i and i + 1
              mirror_chunks(d[0][b2], m0a, m0b);
              mirror_chunks(d[1][b2], m1a, m1b);
              static_for<2>([&](auto rc) {
                constexpr int rr = decltype(rc)::value;      // transposed row c0 + rr
                const uint4& x0 = rr ? m0b : m0a;
                const uint4& x1 = rr ? m1b : m1a;
                const uint4 recv = swap1(sel4(t1, x0, x1));
                TO* q = mrow2 + (32 * (j + b2) + rr) * p.ldc + 32 * i;
                *(uint4*)q = sel4(t1, recv, x0);                      // row c0 - 2 t1 + rr
                *(uint4*)(q + 2 * p.ldc) = sel4(t1, x1, recv);        // row c0 - 2 t1 + 2 + rr
              });
            });
            nst += 16;
          });
        });
        return nst;
      }
      // A^2 + B on a diagonal quadrant: blocks (i, j <= i) in order, the
      // epilogue operand of the next one loaded during this one
      uint2 eb[2][4];
      if (EGROUP) load_e(0, 0, eb[0]);
      static_for<SUB>([&](auto ic) {
        static_for<SUB>([&](auto jc) {
          constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
          if (dq && i < j) return;              // above the diagonal of a diagonal quadrant
          const bool dblk = dq && i == j;
          __builtin_amdgcn_sched_barrier(0);
          constexpr int bq = i * (i + 1) / 2 + j, bb = bq & 1;   // position among blocks j <= i
          if constexpr (EGROUP) {
            if constexpr (j < i) load_e(i, j + 1, eb[bb ^ 1]);
            else if constexpr (i + 1 < SUB) load_e(i + 1, 0, eb[bb ^ 1]);
          }
          uint32_t d[8];
          if constexpr (EGROUP) pack(ic, jc, dblk, d, eb[bb]);
          else pack(ic, jc, dblk, d, epk[EGROUP ? 0 : i][EGROUP ? 0 : j]);
          uint4 wr[2];
          direct_chunks(d, wr);
          const int y0 = 16 * ((lc >> 4) & 1) + 8 * lh;       // block column of the chunk
          static_for<2>([&](auto hc) {
            constexpr int hh = decltype(hc)::value;
            const int r = 16 * hh + (lc & 15);                 // block row of the chunk
            TO* dst = C + (rb0 + 32 * i + r) * p.ldc + cb0 + 32 * j + y0;
            if (!dblk || y0 + 7 <= r) {
              *(uint4*)dst = wr[hh];
            } else if (y0 <= r) {
              union { uint4 v; TO e[8]; } u;
              u.v = wr[hh];
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (y0 + e <= r) dst[e] = u.e[e];
            }
          });
          mirror(ic, jc, dblk, d);
          if (!dblk) nst += 4;
        });
      });
    }
    return nst;
  };

  TileAddr cur, nxt;
  tile_addr(id, cur);
  if (MULTI && nt > 1) tile_addr(id + G, nxt);
  else nxt = cur;
  if constexpr (APPLY) {
    // the first tile's row indices, complete before the first loads of
    // operands are issued (the compiler does not count those)
    load_rows(cur, wr);
#pragma unroll
    for (int i = 0; i < SUB; ++i)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) asm volatile("" : "+v"(wr[i][hh][0]), "+v"(wr[i][hh][1]));
  }
  const int KT = p.K / BK;
  const int GT = nt * KT;                     // stages over all tiles (KT >= NBUF when nt > 1)

  const int pre = GT < NBUF - 1 ? GT : NBUF - 1;
  for (int g = 0; g < pre; ++g)
#pragma unroll
    for (int x = 0; x < 8; ++x) dma(cur.ra, cur.rb, g, g, x);
  wait_vm(8 * (pre - (GT < 2 ? GT : 2)));     // stages 0 and 1 landed
  __syncthreads();

  uint4 fa0[SUB], fb0[SUB], fa1[SUB], fb1[SUB];
#pragma unroll
  for (int i = 0; i < SUB; ++i) { read_a(fa0[i], 0, 0, i); read_b(fb0[i], 0, 0, i, cur.bo); }

  // One stage = 2 k-steps x 4 groups of 4 MFMAs.  Group x of a step issues
  // one DMA instruction of the stage NBUF - 1 ahead (spread out so the vector
  // memory queue never stalls the wave) and reads two fragments of the next
  // k-step (B fragments first), interleaved with its 4 MFMAs.
  int g = 0;                                  // global stage
  int bcur = 0;                               // its LDS buffer, g mod NBUF
  int epi_st = 0;                             // stores of the previous tile's epilogue (per lane)
  // FIRST: a tile's first stage (its first k-step starts the accumulators);
  // LAST: a tile's last stage, which leaves the next stage's fragments unread
  // so that the epilogue runs with them dead (they are read after it)
  // ISS: 1 when the stage NBUF - 1 ahead exists (no test in the loop body),
  // 0 when it does not, 2 to test at run time
  auto stage = [&](auto first_c, auto last_c, auto iss_c, int j, int kt) {
    constexpr bool FIRST = decltype(first_c)::value;
    constexpr bool LAST = decltype(last_c)::value;
    constexpr int ISS = decltype(iss_c)::value;
    // the stage NBUF - 1 ahead: this tile's, or the next tile's first ones
    const bool to_next = MULTI && kt + NBUF - 1 >= KT;
    const bool iss = ISS == 1 || (ISS == 2 && g + NBUF - 1 < GT);
    const int ls = kt + NBUF - 1 >= KT ? kt + NBUF - 1 - KT : kt + NBUF - 1;
    // LDS buffers (global stage mod NBUF, kept as running indices): this
    // stage's, the next stage's, and the look-ahead stage's (the buffer the
    // previous stage used)
    const int bnext = bcur == NBUF - 1 ? 0 : bcur + 1;
    const int ib = bcur == 0 ? NBUF - 1 : bcur - 1;
    int4v ira = cur.ra, irb = cur.rb;
    if (to_next) { ira = nxt.ra; irb = nxt.rb; }
    // B fragments of the next stage: the next tile's after a tile's last stage
    const int bo_next = kt == KT - 1 ? nxt.bo : cur.bo;
    static_for<2 * SUB>([&](auto gxc) {
      constexpr int gx = decltype(gxc)::value;
      constexpr int st = gx / SUB, x = gx % SUB;     // k-step, MFMA row block
      // the group's instructions one by one between its MFMAs (each MFMA
      // holds the matrix pipe for 32 cycles, hiding the issue of what
      // follows it): MFMA, fragment read, MFMA, fragment read, MFMA, DMA,
      // MFMA (measured on MI355X: 3-6 % faster than DMA and reads ahead of
      // the four MFMAs)
      __builtin_amdgcn_sched_barrier(0);
      // fragments of the next k-step: step 1 of this stage, or step 0 of the next stage
      const bool rd = !(LAST && st == 1);
      const int ns = st == 0 ? bcur : bnext;
      const int nst = st == 0 ? 1 : 0;
      uint4 (&na)[SUB] = st == 0 ? fa1 : fa0;
      uint4 (&nb)[SUB] = st == 0 ? fb1 : fb0;
      uint4 (&ca)[SUB] = st == 0 ? fa0 : fa1;
      uint4 (&cbv)[SUB] = st == 0 ? fb0 : fb1;
      auto next_frag = [&](int h) {
        if (!rd) return;
        if (x < 2) read_b(nb[2 * x + h], ns, nst, 2 * x + h, st == 0 ? cur.bo : bo_next);
        else read_a(na[2 * x - 4 + h], ns, nst, 2 * x - 4 + h);
      };
      auto mfma = [&](int jj) {
        const uint4& l = SWAP ? cbv[jj] : ca[x];
        const uint4& r = SWAP ? ca[x] : cbv[jj];
        if (FIRST && st == 0) Mma<T>::first(acc[x][jj], l, r);
        else Mma<T>::run(acc[x][jj], l, r);
      };
      mfma(0);
      __builtin_amdgcn_sched_barrier(0);
      next_frag(0);
      __builtin_amdgcn_sched_barrier(0);
      mfma(1);
      __builtin_amdgcn_sched_barrier(0);
      next_frag(1);
      __builtin_amdgcn_sched_barrier(0);
      mfma(2);
      __builtin_amdgcn_sched_barrier(0);
      if (iss) dma(ira, irb, ls, ib, gx);
      __builtin_amdgcn_sched_barrier(0);
      mfma(3);
    });
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (ISS == 1) {
      // stages g + 3 .. g + NBUF - 1 are issued and may fly on (a constant
      // count), and in a tile's first stages the previous epilogue's stores
      if (MULTI && j > 0 && kt < 2) {
        const int allowed = 8 * (NBUF - 3) + epi_st;
        wait_vm(allowed < 63 ? allowed : 63);
      } else {
        wait_vm(8 * (NBUF - 3));
      }
      stage_barrier();
    } else if (g + 1 < GT) {
      // stage g + 2 must land before this barrier; later stages may fly on,
      // and so may the previous tile's epilogue stores when they were issued
      // after stage g + 2's loads (the first two stages of a tile)
      const int last_issued = g + NBUF - 1 < GT ? g + NBUF - 1 : GT - 1;
      int allowed = g + 2 < GT ? 8 * (last_issued - (g + 2)) : 0;
      if (MULTI && g + 2 < GT && j > 0 && kt < 2) allowed += epi_st;
      wait_vm(allowed < 63 ? allowed : 63);
      stage_barrier();
    }
    ++g;
    bcur = bnext;
  };
  using T1 = std::true_type;
  using T0 = std::false_type;
  using IssYes = std::integral_constant<int, 1>;
  using IssNo = std::integral_constant<int, 0>;
  using IssTest = std::integral_constant<int, 2>;
  for (int j = 0; j < nt; ++j) {
    // a tile's first stage has its look-ahead whenever a tile spans NBUF stages
    if (KT >= NBUF) stage(T1{}, T0{}, IssYes{}, j, 0);
    else stage(T1{}, T0{}, IssTest{}, j, 0);
    // stages whose look-ahead exists: all of a tile followed by another
    // (KT >= NBUF then), else those before the last NBUF - 1
    const int kt_iss = j + 1 < nt ? KT : KT - (NBUF - 1);
    int kt = 1;
    for (; kt < kt_iss; ++kt) stage(T0{}, T0{}, IssYes{}, j, kt);
    for (; kt < KT; ++kt) stage(T0{}, T0{}, IssNo{}, j, kt);
    if constexpr (MULTI) {
      // the finished tile's stores stay in flight while the next tile, whose
      // first stages are already loaded, computes
      if constexpr (SYM) {
        epi_st = epilogue_sym(cur);
      } else {
        epilogue_swap(cur, nxt, j + 1 < nt);
        epi_st = kEpiStores;
        if constexpr (APPLY) {
          static_for<SUB>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            static_for<2>([&](auto hc) {
              constexpr int hh = decltype(hc)::value;
              wr[i][hh][0] = wr_next[i][hh][0];
              wr[i][hh][1] = wr_next[i][hh][1];
            });
          });
        }
      }
      // the next tile's first fragments (after the last tile: an in-bounds
      // read of a buffer no load is writing, unused)
#pragma unroll
      for (int i = 0; i < SUB; ++i) { read_a(fa0[i], bcur, 0, i); read_b(fb0[i], bcur, 0, i, nxt.bo); }
      if (j + 1 < nt) {
        cur = nxt;
        if (j + 2 < nt) tile_addr(id + (j + 2) * G, nxt);
      }
    }
  }

  if constexpr (!MULTI) epilogue_swap(cur, cur, false);
}

// Tiles per work-group for the multi-tile large-tile kernel.  A work-group pays the
// first stages' load latency once and then runs its tiles back to back; with
// T tiles per work-group the launch takes ceil(ceil(n / T) / CUs) rounds of
// T tiles.  The choice minimises rounds x (T x tile + start-up), with a tile
// costing about (KT + 1) stage times and the start-up about 6.
static int compute_units() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

static long long multi_tile_grid(long long ntiles, int KT, int& per_wg) {
  const long long cus = compute_units();
  double best = 0.0;
  per_wg = 1;
  for (int t = 1; t <= 8; ++t) {
    const long long wgs = (ntiles + t - 1) / t;
    const long long rounds = (wgs + cus - 1) / cus;
    const double cost = (double)rounds * ((double)t * (KT + 1) + 6.0);
    if (t == 1 || cost < best) { best = cost; per_wg = t; }
  }
  return (ntiles + per_wg - 1) / per_wg;
}

// The 256 x 256 tile is used for fp16 / bf16 when the shape is a whole
// number of tiles and there are at least 128 of them (half the compute units;
// measured on MI355X, one 4096^2 symmetric product with 136 tiles runs faster
// on them than with 528 tiles of 128 x 128, one 2048^2 product with 36 does
// not); otherwise (ragged shapes, small batches, fp32) the 128 x 128 tile.
static long long tiles_for(const GemmArgs& a, int bm, int& tm, int& tn) {
  tm = (a.M + bm - 1) / bm;
  tn = (a.N + bm - 1) / bm;
  return (long long)(a.op == OP_GEMM ? tm * tn : tm * (tm + 1) / 2) * a.batch;
}

static bool fast_for(const GemmArgs& a, int bm, int es) {
  const int BKE = kRowBytes / es, EPC = 16 / es;
  return a.M % bm == 0 && a.N % bm == 0 && a.K % BKE == 0 && a.lda % EPC == 0 && a.ldb % EPC == 0 &&
         a.ldc % 8 == 0 && aligned16(a.A) && aligned16(a.B) && aligned16(a.C) &&
         (a.batch == 1 || (a.sA % EPC == 0 && a.sB % EPC == 0 && a.sC % 8 == 0)) &&
         (a.E == nullptr || (a.lde % 8 == 0 && aligned16(a.E) && (a.batch == 1 || a.sE % 8 == 0)));
}

bool gemm_large_tile(const GemmArgs& a) {
  if (dtype_size(a.dtype) != 2) return false;
  // the large-tile kernel addresses each operand with 32-bit byte offsets
  const bool fits32 = (long long)a.M * a.lda * 2 < (1LL << 31) &&
                      (long long)(a.op == OP_GEMM ? a.K : a.N) * a.ldb * 2 < (1LL << 31);
  int tm, tn;
  return fits32 && fast_for(a, 256, 2) && tiles_for(a, 256, tm, tn) >= 128;
}

bool gemm_fused_update_ok(const GemmArgs& a) {
  return a.op == OP_GEMM && dtype_size(a.out_dtype) == 2 && gemm_large_tile(a) && a.W && a.idx &&
         a.wlines >= 1 && aligned16(a.W) && (a.batch == 1 || a.sW % 8 == 0);
}

template <typename T, typename TO, int OP, int BM>
static int launch_typed(const GemmArgs& a, hipStream_t s) {
  constexpr bool HALF = sizeof(T) == 2;
  KParams p;
  p.M = a.M; p.N = a.N; p.K = a.K;
  p.A = a.A; p.lda = a.lda; p.sA = a.sA;
  p.B = a.B; p.ldb = a.ldb; p.sB = a.sB;
  p.E = a.E; p.lde = a.lde; p.sE = a.sE;
  p.C = a.C; p.ldc = a.ldc; p.sC = a.sC;
  p.alpha = a.alpha; p.beta = a.beta; p.gamma = a.gamma;
  p.reverse = a.reverse;
  p.same = OP != OP_GEMM && a.A == a.B && a.lda == a.ldb && (a.batch == 1 || a.sA == a.sB);
  p.W = a.W; p.sW = a.sW; p.wlines = a.wlines; p.idx = a.idx;
  p.eta = a.eta; p.u = a.u; p.decay = a.decay;

  int tm, tn;
  const bool big = HALF && gemm_large_tile(a);
  // the fused update: large-tile Q X with 16-byte aligned W rows only
  const bool apply = a.W != nullptr;
  if (apply && (!HALF || !gemm_fused_update_ok(a))) return DION3_ERR_UNSUPPORTED;
  const int bm = big ? 256 : BM;
  const long long grid = tiles_for(a, bm, tm, tn);
  p.tiles_m = tm;
  p.tiles_n = tn;
  p.tiles_per_mat = OP == OP_GEMM ? tm * tn : tm * (tm + 1) / 2;
  if (grid <= 0 || grid > 0x7fffffffLL) return DION3_ERR_UNSUPPORTED;
  p.ntiles = (int)grid;
  p.tiles_per_wg = 1;
  long long wgs = grid;
  if constexpr (sizeof(TO) == 2) {
    if (big && a.K / 32 >= kStages) wgs = multi_tile_grid(grid, a.K / 32, p.tiles_per_wg);
  }

  static const char* names[4] = {"syrk", "sym_sq_add", "sym_mul", "gemm_qx"};
  TimedLaunch tl(apply ? "qx_apply" : names[OP], s);
  if (apply) {
    if constexpr (OP == OP_GEMM && HALF && sizeof(TO) == 2)
      (void)launch((gemm256_kernel<T, TO, OP_GEMM, kStages, true>), dim3((unsigned)wgs), dim3(kThreads), s, p);
  } else if (big) {
    // X X^T without the beta C term is the symmetric product kernel with
    // B = A (same schedule, main loop and epilogue arithmetic; the epilogue
    // operand of beta != 0 costs registers)
    if constexpr (HALF) {
      bool sym_mul_kernel = false;
      if constexpr (OP == OP_SYRK) sym_mul_kernel = a.E == nullptr;
      if constexpr (OP == OP_SYRK)
        if (sym_mul_kernel)
          (void)launch((gemm256_kernel<T, TO, OP_SYM_MUL, kStages>), dim3((unsigned)wgs), dim3(kThreads), s, p);
      if (!sym_mul_kernel)
        (void)launch((gemm256_kernel<T, TO, OP, kStages>), dim3((unsigned)wgs), dim3(kThreads), s, p);
    }
  } else if (fast_for(a, BM, (int)sizeof(T)))
    (void)launch((gemm_kernel<T, TO, OP, false, BM>), dim3((unsigned)grid), dim3(kThreads), s, p);
  else
    (void)launch((gemm_kernel<T, TO, OP, true, BM>), dim3((unsigned)grid), dim3(kThreads), s, p);
  return launch_status();
}

template <int OP>
static int dispatch(const GemmArgs& a, hipStream_t s) {
  constexpr int BM = 128;
  if (a.dtype == DION3_F16) {
    if (a.out_dtype == DION3_F16) return launch_typed<f16, f16, OP, BM>(a, s);
    if constexpr (OP == OP_GEMM)
      if (a.out_dtype == DION3_F32) return launch_typed<f16, float, OP, BM>(a, s);
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
