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
// Accumulation is fp32; the epilogue applies alpha / beta / gamma in fp32 and
// rounds once to the output type.
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


// ---------------------------------------------------------------------------
// Large-tile kernel for fp16 / bf16: a 256 x 256 tile per work-group, 4 waves
// in 2 x 2, each wave owning a 128 x 128 block (4 x 4 MFMA 32x32x16 tiles), so
// every 16-byte fragment read from LDS feeds four MFMAs.  A stage holds 64 K
// elements (128 bytes per row) of both operands, 64 KB; two stages live in LDS.
//
// K-contiguous operands travel from global memory straight into LDS with
// buffer loads that write LDS directly (each lane's 16 bytes land at the
// wave's LDS base + 16 x lane), so no registers are spent on staging: lane L of
// a wave instruction covering rows r0..r0+7 fetches row r = r0 + L/8, the chunk
// whose swizzled position is L mod 8, which puts every chunk in its place.
// The N-contiguous B operand of Q X is instead loaded as 8 x 8 element blocks
// into registers and transposed there, so LDS is always written with 16-byte
// K-contiguous chunks.  MFMA fragments are double-buffered across k-steps so
// LDS latency overlaps the MFMAs of the previous step.
// ---------------------------------------------------------------------------
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

template <typename T>
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
  // in[r] holds elements (r, 0..7); out[c] receives elements (0..7, c)
  uint32_t w[8][4];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    w[r][0] = in[r].x; w[r][1] = in[r].y; w[r][2] = in[r].z; w[r][3] = in[r].w;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t d[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = w[2 * q][c >> 1], b = w[2 * q + 1][c >> 1];
      d[q] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    out[c] = make_uint4(d[0], d[1], d[2], d[3]);
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
// into LDS at `lds` (wave-uniform) + 16 x lane.  Issued from inline assembly
// so that the compiler does not wait for it before unrelated LDS reads: the
// caller waits (vmcnt) before the barrier that publishes the stage.
__device__ __forceinline__ void lds_dma16(const int4v& rsrc, const void* lds, int voffset, int soffset) {
  const int m0 = __builtin_amdgcn_readfirstlane((int)(unsigned)(uintptr_t)
      (const __attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m0), "v"(voffset), "s"(rsrc), "s"(soffset) : "memory", "m0");
}

template <typename T, typename TO, int OP>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm256_kernel(KParams p) {
  constexpr bool SYM = OP != OP_GEMM;
  constexpr bool BT = OP == OP_GEMM;
  constexpr int BM = 256, BN = 256;
  constexpr int BKE = kRowBytes / 2;          // 64 K elements per stage
  constexpr int WT = 128;                     // wave tile edge
  constexpr int SUB = WT / 32;                // 4 x 4 MFMA tiles per wave
  constexpr int ROWS_PER_INSTR = 8;           // 1 KB = 8 LDS rows per wave instruction
  constexpr int INSTR = BM / (4 * ROWS_PER_INSTR);   // 8 instructions per wave per operand

  __shared__ __attribute__((aligned(1024))) char smem[2][2][BM * kRowBytes];

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
  // the tile coordinates are uniform: keep them (and the buffer resources
  // derived from them) in scalar registers
  ti = __builtin_amdgcn_readfirstlane(ti);
  tj = __builtin_amdgcn_readfirstlane(tj);
  const int bu = __builtin_amdgcn_readfirstlane(bat);
  const int m0 = ti * BM, n0 = tj * BN;

  const T* A = (const T*)p.A + bu * p.sA;
  const T* B = (const T*)p.B + bu * p.sB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // direct-to-LDS addressing: this lane fetches row (wave*8 + lane/8) + 32 s of
  // the tile, chunk (lane%8) ^ (lane/8); byte offsets relative to the tile origin
  const int4v ra = make_rsrc(A, (long long)p.M * p.lda * 2);
  const int lrow = wave * ROWS_PER_INSTR + (lane >> 3);
  const int lchunk = (lane & 7) ^ ((lrow >> 1) & 7);   // rows r0 + 32 s keep (row/2) mod 8
  const int va = ((m0 + lrow) * (int)p.lda + lchunk * 8) * 2;
  const int rstep_a = 4 * ROWS_PER_INSTR * (int)p.lda * 2;   // 32 rows
  const int4v rb = make_rsrc(B, BT ? (long long)p.K * p.ldb * 2 : (long long)p.N * p.ldb * 2);
  const int vb = ((n0 + lrow) * (int)p.ldb + lchunk * 8) * 2;
  const int rstep_b = 4 * ROWS_PER_INSTR * (int)p.ldb * 2;
  // Q X: the N-contiguous B operand is read with ordinary buffer loads into
  // registers (the compiler tracks them); this lane's 8 x 8 block starts at
  // row 8 kb, column n0 + 8 nb of the stage
  const __amdgpu_buffer_rsrc_t rbq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(B), 0, (int)(BT ? min((long long)p.K * p.ldb * 2, 0x7fffffffLL) : 0), 0x00020000);
  const int vbt = ((tid & 7) * 8 * (int)p.ldb + n0 + (tid >> 3) * 8) * 2;
  (void)rb; (void)vb; (void)rstep_b; (void)rbq; (void)vbt;

  floatx16 acc[SUB][SUB];
#pragma unroll
  for (int i = 0; i < SUB; ++i)
#pragma unroll
    for (int j = 0; j < SUB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 rbt[8];   // transposed-B staging (Q X only)

  auto issue_stage = [&](int buf, int k0) {
    char* sa = smem[buf][0] + wave * ROWS_PER_INSTR * kRowBytes;
#pragma unroll
    for (int s = 0; s < INSTR; ++s) lds_dma16(ra, sa + s * 4 * ROWS_PER_INSTR * kRowBytes, va, k0 * 2 + s * rstep_a);
    if (!BT) {
      char* sb = smem[buf][1] + wave * ROWS_PER_INSTR * kRowBytes;
#pragma unroll
      for (int s = 0; s < INSTR; ++s) lds_dma16(rb, sb + s * 4 * ROWS_PER_INSTR * kRowBytes, vb, k0 * 2 + s * rstep_b);
    } else {
      // an 8 (K) x 8 (N) block per thread (kb = tid mod 8, nb = tid / 8): rows
      // k0 + 8 kb + r, columns n0 + 8 nb + c; eight consecutive lanes share
      // nb, so each LDS write instruction fills whole 128-byte rows
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rbq, vbt, (k0 + r) * (int)p.ldb * 2, 0);
        rbt[r] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    }
  };
  auto finish_stage = [&](int buf) {
    if (BT) {
      char* sb = smem[buf][1];
      const int kb = tid & 7, nb = tid >> 3;
      uint4 tr[8];
      transpose8x8<T>(rbt, tr);
#pragma unroll
      for (int c = 0; c < 8; ++c) *(uint4*)(sb + swz(nb * 8 + c, kb)) = tr[c];
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  const int KT = p.K / BKE;
  issue_stage(0, 0);
  finish_stage(0);

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) issue_stage(cur ^ 1, (kt + 1) * BKE);
    const char* sa = smem[cur][0];
    const char* sb = smem[cur][1];
    // every fragment of the stage gets its own registers (32 x 16 bytes per
    // lane), so reads for the next k-step can be in flight during this one
    constexpr int STEPS = kChunks / 2;
    uint4 fa[STEPS][SUB], fb[STEPS][SUB];
    static_for<STEPS>([&](auto sc) {
      constexpr int st = decltype(sc)::value;
      const int chunk = 2 * st + (lane >> 5);
#pragma unroll
      for (int i = 0; i < SUB; ++i) fa[st][i] = *(const uint4*)(sa + swz(wm * WT + i * 32 + (lane & 31), chunk));
#pragma unroll
      for (int j = 0; j < SUB; ++j) fb[st][j] = *(const uint4*)(sb + swz(wn * WT + j * 32 + (lane & 31), chunk));
    });
    static_for<STEPS>([&](auto sc) {
      constexpr int st = decltype(sc)::value;
#pragma unroll
      for (int i = 0; i < SUB; ++i)
#pragma unroll
        for (int j = 0; j < SUB; ++j) Mma<T>::run(acc[i][j], fa[st][i], fb[st][j]);
    });
    // schedule: step 0's reads, then each step's MFMAs with the next step's
    // reads interleaved (one read per two MFMAs)
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * SUB, 0);
    static_for<(STEPS - 1) * 2 * SUB>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    });
    __builtin_amdgcn_sched_group_barrier(0x008, SUB * SUB, 0);
    if (kt + 1 < KT) finish_stage(cur ^ 1);
  }

  // ---- epilogue: the lower triangle and its mirror; diagonal tiles write
  // every entry exactly once (i >= j directly, i > j mirrored)
  TO* C = (TO*)p.C + bu * p.sC;
  const TO* E = (const TO*)p.E + (p.E ? bu * p.sE : 0);
  const bool diag_tile = SYM && ti == tj;
  if (diag_tile && wm < wn) return;            // the upper quadrant mirrors the lower one
  constexpr bool HAS_E = OP == OP_SQ_ADD || OP == OP_SYRK;
  const bool use_e = OP == OP_SQ_ADD || (OP == OP_SYRK && p.beta != 0.f);
  // The epilogue operand is symmetric, so the four values E[gi..gi+3][gj] this
  // lane needs per group are E[gj][gi..gi+3]: one 8-byte load.  All of them are
  // issued before any store (the memory counter also counts stores).
  uint2 epk[SUB][SUB][4];
  if constexpr (HAS_E) {
    if (use_e) {
      static_for<SUB>([&](auto ic) {
        static_for<SUB>([&](auto jc) {
          constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
          const int gi0 = m0 + wm * WT + i * 32;
          const int gj0 = n0 + wn * WT + j * 32;
          if (gi0 < gj0) return;
          const int gj = gj0 + (lane & 31);
          static_for<4>([&](auto gc) {
            constexpr int g = decltype(gc)::value;
            const int gib = gi0 + 8 * g + 4 * (lane >> 5);
            epk[i][j][g] = *(const uint2*)(E + (long long)gj * p.lde + gib);
          });
        });
      });
    }
  }
  asm volatile("" ::: "memory");
  static_for<SUB>([&](auto ic) {
    static_for<SUB>([&](auto jc) {
      constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
      const int gi0 = m0 + wm * WT + i * 32;
      const int gj0 = n0 + wn * WT + j * 32;
      if (SYM && gi0 < gj0) return;            // above the diagonal (diagonal tiles only)
      const bool below = !SYM || gi0 > gj0;    // whole 32 x 32 block strictly below
      const int gj = gj0 + (lane & 31);
      static_for<4>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        const int gib = gi0 + 8 * g + 4 * (lane >> 5);
        union { uint2 u; TO e[4]; } ev;
        if constexpr (HAS_E) ev.u = epk[i][j][g];
        TO vv[4];
        static_for<4>([&](auto qc) {
          constexpr int q = decltype(qc)::value;
          const int gi = gib + q;
          float v = p.alpha * acc[i][j][4 * g + q];
          if constexpr (HAS_E) {
            if (use_e) v += p.beta * Store<TO>::to_f32(ev.e[q]);
          }
          if (OP == OP_SQ_ADD && gi == gj) v += p.gamma;
          vv[q] = Store<TO>::from_f32(v);
          if (below || gi >= gj) C[(long long)gi * p.ldc + gj] = vv[q];
        });
        if (SYM) {
          if (below) {
            // C[gj][gib .. gib+3]: four consecutive elements, one 8-byte store
            union { uint2 u; TO e[4]; } pk;
            static_for<4>([&](auto qc) { pk.e[decltype(qc)::value] = vv[decltype(qc)::value]; });
            *(uint2*)(C + (long long)gj * p.ldc + gib) = pk.u;
          } else {
            static_for<4>([&](auto qc) {
              constexpr int q = decltype(qc)::value;
              if (gib + q > gj) C[(long long)gj * p.ldc + gib + q] = vv[q];
            });
          }
        }
      });
    });
  });
}

template <typename T, typename TO, int OP, int BM>
static int launch_typed(const GemmArgs& a, hipStream_t s) {
  constexpr int BKE = kRowBytes / (int)sizeof(T);
  constexpr int EPC = Mma<T>::EPC;
  constexpr bool HALF = sizeof(T) == 2;
  KParams p;
  p.M = a.M; p.N = a.N; p.K = a.K;
  p.A = a.A; p.lda = a.lda; p.sA = a.sA;
  p.B = a.B; p.ldb = a.ldb; p.sB = a.sB;
  p.E = a.E; p.lde = a.lde; p.sE = a.sE;
  p.C = a.C; p.ldc = a.ldc; p.sC = a.sC;
  p.alpha = a.alpha; p.beta = a.beta; p.gamma = a.gamma;

  // The 256 x 256 tile is used for fp16 / bf16 when the shape is a whole
  // number of tiles and there are at least two tiles per compute unit;
  // otherwise (ragged shapes, small batches, fp32) the 128 x 128 tile.
  auto tiles_for = [&](int bm, int& tm, int& tn) {
    tm = (a.M + bm - 1) / bm;
    tn = (a.N + bm - 1) / bm;
    return (long long)(OP == OP_GEMM ? tm * tn : tm * (tm + 1) / 2) * a.batch;
  };
  auto fast_for = [&](int bm) {
    return a.M % bm == 0 && a.N % bm == 0 && a.K % BKE == 0 && a.lda % EPC == 0 &&
           a.ldb % EPC == 0 && a.ldc % 8 == 0 && aligned16(a.A) && aligned16(a.B) &&
           aligned16(a.C) && (a.batch == 1 || (a.sA % EPC == 0 && a.sB % EPC == 0 && a.sC % 8 == 0)) &&
           (a.E == nullptr || (a.lde % 8 == 0 && aligned16(a.E) && (a.batch == 1 || a.sE % 8 == 0)));
  };
  int tm, tn;
  const bool big = HALF && fast_for(256) && tiles_for(256, tm, tn) >= 512;
  const int bm = big ? 256 : BM;
  const long long grid = tiles_for(bm, tm, tn);
  p.tiles_m = tm;
  p.tiles_n = tn;
  p.tiles_per_mat = OP == OP_GEMM ? tm * tn : tm * (tm + 1) / 2;
  if (grid <= 0 || grid > 0x7fffffffLL) return DION3_ERR_UNSUPPORTED;

  static const char* names[4] = {"syrk", "sym_sq_add", "sym_mul", "gemm_qx"};
  TimedLaunch tl(names[OP], s);
  if (big) {
    if constexpr (HALF)
      hipLaunchKernelGGL((gemm256_kernel<T, TO, OP>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  } else if (fast_for(BM))
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
