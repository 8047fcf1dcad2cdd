// bf16 MFMA GEMM with an activation epilogue: the MLP form of the chain.
//
// METP article (abstract): O = f(A.B).C with f between two consecutive
// products; for the MLP, A = X, B = W1, f = GeLU, C = W2 (TSP article, "Lo que
// realmente significa plegar": one weight shard of the MLP ring).  This kernel
// computes one product C = act(A.B) with A [M, K] and B [K, N] row-major; the
// MLP runs it twice (act = GeLU into the workspace, then act = identity).
//
// bf16: tile 256 x 256 x 64 per 512-thread workgroup (8 waves, 2 per SIMD),
// 2 x 4 waves of 128 x 64, each a 4 x 2 grid of v_mfma_f32_32x32x16_bf16 blocks
// with f32 accumulation.  A and B tiles are staged row-major in LDS,
// double-buffered through registers (one global fetch in flight while the
// previous tile is consumed); the A operand is a plain 16-byte LDS read (8
// consecutive k of one row, pitch BK + 8 so the reads of a wave spread over
// all banks), the B operand (8 consecutive k of one column) comes from
// ds_read_b64_tr_b16 at pitch BN + 32.  Rows/columns past M/N and k past K are
// zero-filled.  The f32 path for f32 inputs keeps a 128 x 128 x 32 tile per
// 256 threads with v_mfma_f32_32x32x2_f32.
#include "internal.h"

namespace chain {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int TM = 128, TN = 128, TK = 32;
constexpr int LDA = TK + 8;     // A tile pitch (elements)
constexpr int LDB = TN + 8;     // B tile pitch (elements)

__device__ inline i16x4 ds_read_tr(const __bf16 *p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

__device__ inline float activate(float z, int act) {
  if (act == CHAIN_ACT_GELU_ERF) return 0.5f * z * (1.f + erff(z * 0.70710678118654752f));
  if (act == CHAIN_ACT_GELU_TANH) {
    const float u = 0.79788456080286536f * (z + 0.044715f * z * z * z);
    return 0.5f * z * (1.f + tanhf(u));
  }
  return z;
}

// bf16 path: 256 x 256 x 64 block tiles over eight waves (two per SIMD), each
// wave computing 128 x 64 of C as 4 x 2 blocks of 32 x 32.  Every A fragment
// read from LDS feeds two MFMAs and every B fragment four (0.75 KB of LDS reads
// per MFMA).  A/B tiles are double-buffered in LDS; the global loads of stage
// k+1 are in flight while stage k is computed, and within a stage the
// fragments of k-step s+1 are read while the MFMAs of k-step s issue.
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WTM = 128, WTN = 64;        // wave tile
constexpr int MB = WTM / 32, NB = WTN / 32;
constexpr int LDAB = BK + 8;              // A pitch: conflict-free 16-byte reads
constexpr int LDBB = BN + 32;             // B pitch: conflict-free transposing reads
constexpr int GLOADS = BM * BK / 8 / 512; // 16-byte chunks per thread per operand

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2)))
void gemm_bf16_kernel(const GemmParams p) {
  static_assert(BM * BK == BK * BN, "A and B stages split the same way");
  __shared__ __attribute__((aligned(16))) __bf16 as[2][BM * LDAB];
  __shared__ __attribute__((aligned(16))) __bf16 bs[2][BK * LDBB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h2 = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 2, wn = wave & 3;

  const int tiles_n = (p.N + BN - 1) / BN;
  const int tiles = ((p.M + BM - 1) / BM) * tiles_n;
  const int tile = xcd_remap(blockIdx.x, tiles);
  const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;

  const __bf16 *A = (const __bf16 *)p.a;
  const __bf16 *B = (const __bf16 *)p.b;
  uint4 ar[GLOADS], br[GLOADS];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < GLOADS; ++i) {
      const int c = tid + 512 * i;
      const int ra = c >> 3, ka = (c & 7) * 8;            // A: 256 rows x 8 chunks
      const int gm = m0 + ra, gk = k0 + ka;
      ar[i] = (gm < p.M && gk < p.K) ? *(const uint4 *)(A + (int64_t)gm * p.lda + gk)
                                     : make_uint4(0, 0, 0, 0);
      const int kb = c >> 5, nb = (c & 31) * 8;           // B: 64 rows x 32 chunks
      const int gk2 = k0 + kb, gn = n0 + nb;
      br[i] = (gk2 < p.K && gn < p.N) ? *(const uint4 *)(B + (int64_t)gk2 * p.ldb + gn)
                                      : make_uint4(0, 0, 0, 0);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < GLOADS; ++i) {
      const int c = tid + 512 * i;
      *(uint4 *)(&as[buf][(c >> 3) * LDAB + (c & 7) * 8]) = ar[i];
      *(uint4 *)(&bs[buf][(c >> 5) * LDBB + (c & 31) * 8]) = br[i];
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

  const int trow = (lane & 15) >> 2;
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto frags = [&](int buf, int ks, bf16x8 (&a)[MB], bf16x8 (&b)[NB]) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
      a[i] = *(const bf16x8 *)(&as[buf][(wm * WTM + i * 32 + l32) * LDAB + ks * 16 + 8 * h2]);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const __bf16 *src = &bs[buf][(ks * 16 + 8 * h2 + trow) * LDBB + wn * WTN + j * 32 + tcol];
      const i16x4 lo = ds_read_tr(src);
      const i16x4 hi = ds_read_tr(src + 4 * LDBB);
      b[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  const int nk = (p.K + BK - 1) / BK;
  gload(0);
  swrite(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) gload((kt + 1) * BK);
    bf16x8 a0[MB], b0[NB], a1[MB], b1[NB];
    frags(buf, 0, a0, b0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ks += 2) {
      frags(buf, ks + 1, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 2 < BK / 16) frags(buf, ks + 2, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b1[j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) swrite(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane owns column l32 of each 32x32 block, rows 8*(r/4) + 4*h2 + r%4
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int gn = n0 + wn * WTN + j * 32 + l32;
      if (gn >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
        if (gm >= p.M) continue;
        const float v = activate(acc[i][j][r], p.act);
        if (p.c_f32) ((float *)p.c)[(int64_t)gm * p.ldc + gn] = v;
        else ((__bf16 *)p.c)[(int64_t)gm * p.ldc + gn] = (__bf16)v;
      }
    }
}

// f32 inputs: same tiles on v_mfma_f32_32x32x2_f32 (A: lane holds A[m][k0 + h2],
// B: lane holds B[k0 + h2][n]); exact f32 products, f32 accumulation.
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmParams p) {
  __shared__ float as[TM][TK + 1];
  __shared__ float bs[TK][TN + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h2 = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (p.N + TN - 1) / TN;
  const int tiles = ((p.M + TM - 1) / TM) * tiles_n;
  const int tile = xcd_remap(blockIdx.x, tiles);
  const int m0 = (tile / tiles_n) * TM, n0 = (tile % tiles_n) * TN;
  const float *A = (const float *)p.a;
  const float *B = (const float *)p.b;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  for (int k0 = 0; k0 < p.K; k0 += TK) {
    for (int e = tid; e < TM * TK; e += 256) {
      const int r = e / TK, c = e % TK;
      as[r][c] = (m0 + r < p.M && k0 + c < p.K) ? A[(int64_t)(m0 + r) * p.lda + k0 + c] : 0.f;
    }
    for (int e = tid; e < TK * TN; e += 256) {
      const int r = e / TN, c = e % TN;
      bs[r][c] = (k0 + r < p.K && n0 + c < p.N) ? B[(int64_t)(k0 + r) * p.ldb + n0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < TK; kk += 2) {
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = as[wm * 64 + i * 32 + l32][kk + h2];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = bs[kk + h2][wn * 64 + j * 32 + l32];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gn = n0 + wn * 64 + j * 32 + l32;
      if (gn >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
        if (gm >= p.M) continue;
        const float v = activate(acc[i][j][r], p.act);
        if (p.c_f32) ((float *)p.c)[(int64_t)gm * p.ldc + gn] = v;
        else ((__bf16 *)p.c)[(int64_t)gm * p.ldc + gn] = (__bf16)v;
      }
    }
}

}  // namespace

hipError_t launch_gemm(const GemmParams &p, int dtype, hipStream_t stream) {
  if (dtype == CHAIN_BF16) {
    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3(tiles), dim3(512), 0, stream, p);
  } else {
    const int tiles = ((p.M + TM - 1) / TM) * ((p.N + TN - 1) / TN);
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(tiles), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace chain
