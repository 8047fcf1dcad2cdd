// bf16 MFMA GEMM with an activation epilogue: the MLP form of the chain.
//
// METP article (abstract): O = f(A.B).C with f between two consecutive
// products; for the MLP, A = X, B = W1, f = GeLU, C = W2 (TSP article, "Lo que
// realmente significa plegar": one weight shard of the MLP ring).  This kernel
// computes one product C = act(A.B) with A [M, K] row-major and B [K, N] in
// either layout (n contiguous, or k contiguous: the transpose of a row-major
// [N, K] weight, as linear layers store it); the MLP runs it twice (act = GeLU
// into the workspace, then act = identity).
//
// bf16: one workgroup per CU computes a 256 x BN tile (BN = 352, 256, 192 or
// 128, picked per launch so the tiles fill whole rounds of the chip with the
// least padding) on v_mfma_f32_32x32x16_bf16 blocks with f32 accumulators, as
// 4 x 2 waves of 64 x BN/2 (two waves per SIMD).  Operands are swapped in the
// MFMA (it computes the transposed block) so a lane ends up holding four
// consecutive output columns of one row: 8-byte stores.  Buffer loads that
// write LDS directly fill a ring of k-stages (four of 32 k, or two of 64 k for
// the 256- and 352-wide tiles), rows XOR-swizzled instead of padded, and
// fragments are streamed a few MFMAs ahead of use:
//  - gemm_bf16_w8r_kernel_NB: k-contiguous B, staged like A (B rows are
//    output columns), read with 16-byte LDS reads;
//  - gemm_bf16_w8rt_kernel_NB: n-contiguous B, staged by k row and read with
//    ds_read_b64_tr_b16 (the transposing read gives the same operand);
//  - gemm_bf16_w8_gated_kernel_NBW / gemm_bf16_w8t_gated_kernel_NBW: the gated
//    MLP's first product (TSP article: gate and up projection shards), two B
//    matrices whose tiles share the A tile, act(gate) times up in the epilogue;
//  - fallbacks for operands whose tile rows span 2 GiB or more (beyond 32-bit
//    buffer offsets): gemm_bf16_dtl_kernel_NBW (four waves of 128 x BN/2, the
//    same ring, k-contiguous B) and gemm_bf16_kernel<NBW> (k-tiles of 64 staged
//    through registers into two LDS buffers, n-contiguous B).
// Every path gives the same MFMA operands in the same k order, so the weight
// layouts and paths give the same bits.  The f32 path for f32 inputs keeps a
// 128 x 128 x 32 tile per 256 threads with v_mfma_f32_32x32x2_f32.
#include "internal.h"

#include <type_traits>

namespace chain {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 128, TN = 128, TK = 32;   // f32 path

// Transposing LDS read (in each group of 16 lanes, lane i receives element i % 4
// of the 4-element rows addressed by lanes 4e + i / 4, e = 0..3).  The restrict
// qualifier gives the inlined read alias-scope information; without it the
// compiler cannot tell it from direct-to-LDS loads in flight and waits for all
// of them (vmcnt(0)) before it.  Every stage a read touches has landed and
// passed a barrier.
__device__ inline i16x4 ds_read_tr(const __bf16 *__restrict__ p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26 (after Hastings): erf(x) = 1 - t (a1 + a2 t + ... + a5 t^4) exp(-x^2),
// t = 1 / (1 + p x) for x >= 0, odd in x; absolute error at most 1.5e-7.  One
// reciprocal and one exp2 instead of a general-purpose erff, which matters in
// an epilogue no other wave can overlap.
__device__ inline float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.f));
  float q = fmaf(t, 1.061405429f, -1.453152027f);
  q = fmaf(t, q, 1.421413741f);
  q = fmaf(t, q, -0.284496736f);
  q = fmaf(t, q, 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * ax * ax);
  return copysignf(fmaf(-q * t, e, 1.f), x);
}

__device__ inline float activate(float z, int act) {
  if (act == CHAIN_ACT_GELU_ERF) return 0.5f * z * (1.f + erf_as(z * 0.70710678118654752f));
  if (act == CHAIN_ACT_GELU_TANH) {
    const float u = 0.79788456080286536f * (z + 0.044715f * z * z * z);
    return 0.5f * z * (1.f + tanhf(u));
  }
  if (act == CHAIN_ACT_SILU) return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
  return z;
}

constexpr int BM = 256, BK = 64;
constexpr int LDA = BK + 8;        // pitch of k-contiguous stages

__device__ inline u32x4 ld16(const __bf16 *p) { return *(const u32x4 *)p; }

// Epilogue of a wave's MI x NBW grid of 32 x 32 blocks (rows r0 + 32 i + l32,
// columns c0 + 32 j + 8 (r / 4) + 4 h2 + r % 4 in element r of acc[i][j]):
// act(), then stores.  GATED: blocks 2j and 2j + 1 are the gate and up
// products of output block j, which takes act(gate) * up.  bf16 rows that allow it take 16-byte stores: the two
// lane halves (same row) swap half of their 4-column groups, so that each lane
// holds 8 consecutive columns (half 0: 8g..8g+7, half 1: 8(g+1)..8(g+1)+7, for
// g = 0, 2); otherwise 4 columns at a time.
template <int MI, int NBW, bool GATED, int ACT>
__device__ __forceinline__ void gemm_store_tile(const GemmParams &p, const f32x16 (&acc)[MI][NBW], int r0,
                                                int c0, int l32, int h2) {
  constexpr int NOB = GATED ? NBW / 2 : NBW;   // 32-column output blocks
  const bool vec16 = !p.c_f32 && ((uintptr_t)p.c % 16 == 0) && (p.ldc % 8 == 0);
  auto pack2 = [](float x, float y) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 w = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, w);
  };
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int gm = r0 + i * 32 + l32;   // the same in both lane halves
    if (gm >= p.M) continue;
#pragma unroll
    for (int j = 0; j < NOB; ++j) {
      f32x16 v;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        v[r] = GATED ? activate(acc[i][2 * j][r], ACT) * acc[i][2 * j + 1][r] : activate(acc[i][j][r], ACT);
      const int col0 = c0 + j * 32;
      if (vec16) {
#pragma unroll
        for (int g = 0; g < 4; g += 2) {
          const auto x0 = __builtin_amdgcn_permlane32_swap(pack2(v[4 * g], v[4 * g + 1]),
                                                           pack2(v[4 * g + 4], v[4 * g + 5]), false, false);
          const auto x1 = __builtin_amdgcn_permlane32_swap(pack2(v[4 * g + 2], v[4 * g + 3]),
                                                           pack2(v[4 * g + 6], v[4 * g + 7]), false, false);
          const int gn = col0 + 8 * (g + h2);
          if (gn < p.N)
            *(u32x4 *)((__bf16 *)p.c + (int64_t)gm * p.ldc + gn) = u32x4{x0[0], x1[0], x0[1], x1[1]};
        }
      } else {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int gn = col0 + 8 * r4 + 4 * h2;
          if (gn >= p.N) continue;   // N % 4 == 0: the four columns are all in or all out
          const f32x4 w4 = {v[4 * r4], v[4 * r4 + 1], v[4 * r4 + 2], v[4 * r4 + 3]};
          const int64_t off = (int64_t)gm * p.ldc + gn;
          if (p.c_f32) {
            float *c = (float *)p.c + off;
            if (p.c_vec) *(f32x4 *)c = w4;
            else c[0] = w4[0], c[1] = w4[1], c[2] = w4[2], c[3] = w4[3];
          } else {
            __bf16 *c = (__bf16 *)p.c + off;
            const bf16x4 w = {(__bf16)w4[0], (__bf16)w4[1], (__bf16)w4[2], (__bf16)w4[3]};
            if (p.c_vec) *(bf16x4 *)c = w;
            else c[0] = w[0], c[1] = w[1], c[2] = w[2], c[3] = w[3];
          }
        }
      }
    }
  }
}

// n-contiguous B (row-major [K, N] weights).  NBW = 32-column blocks per wave
// (BN = 64 * NBW).  ACT: the epilogue's activation, one instantiation each (a
// run-time choice among several epilogues costs registers in the main loop).
// Eight waves (two per SIMD) of 64 x BN/2 share the tile.  k-tiles of 64 are
// staged through registers into two LDS buffers (A as [256][64 + 8], B as
// [64][BN' + 32] read with ds_read_b64_tr_b16); the fetch of tile k+2 is issued
// once tile k+1 is written to LDS.
template <int NBW, int ACT>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_kernel(const GemmParams p) {
  constexpr int NW = 8, NT = 64 * NW;                    // waves, threads
  constexpr int WMR = BM / (NW / 2), MI = WMR / 32;      // rows per wave, 32-row blocks per wave
  constexpr int BN = 64 * NBW, WTN = 32 * NBW;
  constexpr int LDBN = ((BN + 127) / 128) * 128 + 32;   // B pitch: conflict-free tr reads
  constexpr int BSZ = BK * LDBN;
  constexpr int AL = BM * BK / 8 / NT;                   // 16-byte chunks per thread
  constexpr int BL = BN * BK / 8 / NT;
  constexpr int BCH = BN / 8;                            // chunks per B row
  __shared__ __attribute__((aligned(16))) __bf16 as[2][BM * LDA];
  __shared__ __attribute__((aligned(16))) __bf16 bs[2][BSZ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h2 = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;

  // Tile order: groups of 4 row blocks x all column blocks, row block fastest,
  // so the 32 tiles an XCD runs at once cover 4 x 8 blocks.
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int t = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  constexpr int GM = 4;
  const int g = t / (GM * tiles_n), fm = g * GM;
  const int gmn = min(GM, tiles_m - fm), loc = t - g * GM * tiles_n;
  const int m0 = (fm + loc % gmn) * BM, n0 = (loc / gmn) * BN;
  const __bf16 *A = (const __bf16 *)p.a;
  const __bf16 *B = (const __bf16 *)p.b;
  const int64_t ldb = p.b_sk;
  const int nk = (p.K + BK - 1) / BK;
  const int nk_plain = (m0 + BM <= p.M && n0 + BN <= p.N) ? p.K / BK : 0;

  // Chunk c = tid + NT i of a stage: A row (c >> 3) = (tid >> 3) + (NT / 8) i, k
  // chunk c & 7 = tid & 7; a B row holds BCH chunks.  Per-thread byte offsets
  // stay 32-bit; the per-i part is uniform.
  const char *Ab = (const char *)A, *Bb = (const char *)B;
  const uint32_t a_off = (uint32_t)((tid >> 3) * p.lda + (tid & 7) * 8) * 2u;
  const uint32_t b_off = (uint32_t)((tid / BCH) * ldb + (tid % BCH) * 8) * 2u;
  u32x4 ar[AL], br[BL];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
    if (kt < nk_plain) {
#pragma unroll
      for (int i = 0; i < AL; ++i) {
        const char *base = Ab + ((int64_t)(m0 + (NT / 8) * i) * p.lda + k0) * 2;
        ar[i] = *(const u32x4 *)(base + a_off);
      }
#pragma unroll
      for (int i = 0; i < BL; ++i) {
        const int c = tid + NT * i;
        if (NT % BCH == 0) {
          const char *base = Bb + ((int64_t)(k0 + (NT / BCH) * i) * ldb + n0) * 2;
          br[i] = *(const u32x4 *)(base + b_off);
        } else {
          br[i] = ld16(B + (int64_t)(k0 + c / BCH) * ldb + n0 + (c % BCH) * 8);
        }
      }
    } else {
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < AL; ++i) {
        const int c = tid + NT * i;
        const int gm = m0 + (c >> 3), gk = k0 + (c & 7) * 8;
        const bool ok = gm < p.M && gk < p.K;
        const u32x4 v = ld16(ok ? A + (int64_t)gm * p.lda + gk : A);
        ar[i] = ok ? v : z;
      }
#pragma unroll
      for (int i = 0; i < BL; ++i) {
        const int c = tid + NT * i;
        const int gk = k0 + c / BCH, gn = n0 + (c % BCH) * 8;
        const bool ok = gk < p.K && gn < p.N;
        const u32x4 v = ld16(ok ? B + (int64_t)gk * ldb + gn : B);
        br[i] = ok ? v : z;
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int c = tid + NT * i;
      *(u32x4 *)(&as[buf][(c >> 3) * LDA + (c & 7) * 8]) = ar[i];
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int c = tid + NT * i;
      *(u32x4 *)(&bs[buf][(c / BCH) * LDBN + (c % BCH) * 8]) = br[i];
    }
  };

  struct Frags {
    bf16x8 a[MI], b[NBW];
  };
  const int trow = (lane & 15) >> 2;
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto frags = [&](int buf, int ks, Frags &f) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
      f.a[i] = *(const bf16x8 *)(&as[buf][(wm * WMR + i * 32 + l32) * LDA + ks * 16 + 8 * h2]);
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const __bf16 *src = &bs[buf][(ks * 16 + 8 * h2 + trow) * LDBN + wn * WTN + j * 32 + tcol];
      const i16x4 lo = ds_read_tr(src);
      const i16x4 hi = ds_read_tr(src + 4 * LDBN);
      f.b[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  // acc[i][j] holds the transposed 32 x 32 block: lane (h2, l32) has row
  // m = l32 and columns n = 8 * (r / 4) + 4 * h2 + r % 4 in element r.
  f32x16 acc[MI][NBW];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = f32x16{};
  auto mfmas = [&](const Frags &f) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  };

  Frags f0;
  if (nk > 0) {   // K = 0: nothing to load (the operands may have no storage)
    gload(0);
    swrite(0);
    if (nk > 1) gload(1);
    __syncthreads();
  }
  if constexpr (NBW == 4) {
    // One fragment set per wave (the other wave on the SIMD covers the read
    // latency), which keeps the 64 x 256 wave tile within 256 registers.
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1, nxt = cur ^ 1;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        frags(cur, ks, f0);
        mfmas(f0);
        if (ks == 1 && kt + 1 < nk) {
          swrite(nxt);
          if (kt + 2 < nk) gload(kt + 2);
        }
      }
      __syncthreads();
    }
  } else {
    // Narrower tiles leave room for two fragment sets: each k-step's fragments
    // are read while the previous k-step's MFMAs run.
    Frags f1;
    if (nk > 0) frags(0, 0, f0);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1, nxt = cur ^ 1;
      frags(cur, 1, f1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(f0);
      __builtin_amdgcn_sched_barrier(0);
      frags(cur, 2, f0);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(f1);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < nk) {
        swrite(nxt);
        if (kt + 2 < nk) gload(kt + 2);
      }
      frags(cur, 3, f1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(f0);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      if (kt + 1 < nk) frags(nxt, 0, f0);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(f1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  gemm_store_tile<MI, NBW, false, ACT>(p, acc, m0 + wm * WMR, n0 + wn * WTN, l32, h2);
}

// ---- k-contiguous A and B: direct-to-LDS stage ring ------------------------
//
// Same 256 x BN tile, waves and MFMA blocks as above, but the operands never
// pass through registers: each wave-level global_load_lds_dwordx4 drops 64
// lanes x 16 bytes (16 rows x 32 k) straight into LDS.  k-tiles of 32 sit in
// a ring of four stages and are fetched three stages ahead, so 3 x (256 + BN)
// x 64 bytes per CU are in flight while a stage is computed.  A row of a stage
// is 64 bytes (four 16-byte chunks); chunk c of row r is stored at position
// c ^ ((r >> 2) & 3), which puts the 16-byte fragment reads of 16 consecutive
// rows on 16 distinct bank groups (the load side chooses which global chunk
// each lane fetches, so the swizzle costs nothing).  Rows past M or N read the
// last valid row (their results are never stored); chunks past K read a valid
// chunk and are overwritten with zeros once they have landed.
constexpr int DBK = 32;   // k per stage
constexpr int DST = 4;    // stages in the ring

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// GATED: the BN staged B rows of a tile are BN/2 output columns of B (gate) and
// the same BN/2 columns of B2 (up), arranged so that each wave's 32-row blocks
// alternate gate, up for the same 32 columns: the epilogue then finds the two
// products of an output element in the same lane and register.
template <int NBW, bool GATED, int ACT>
__device__ __forceinline__ void gemm_bf16_dtl(const GemmParams &p) {
  constexpr int BN = 64 * NBW, WTN = 32 * NBW;
  constexpr int OBN = GATED ? BN / 2 : BN;   // output columns per tile
  static_assert(!GATED || NBW % 2 == 0, "gated tiles pair 32-row blocks");
  constexpr int A_BYTES = BM * DBK * 2, B_BYTES = BN * DBK * 2, STAGE = A_BYTES + B_BYTES;
  constexpr int LA = 4, LB = NBW, L = LA + LB;   // 1 KB loads per wave per stage
  __shared__ __attribute__((aligned(1024))) char lds[DST * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;

  // Tile order: groups of 4 row blocks x all column blocks, row block fastest,
  // so the 32 tiles an XCD runs at once cover 4 x 8 blocks.
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + OBN - 1) / OBN;
  const int t = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  constexpr int GM = 4;
  const int g = t / (GM * tiles_n), fm = g * GM;
  const int gmn = min(GM, tiles_m - fm), loc = t - g * GM * tiles_n;
  const int m0 = (fm + loc % gmn) * BM, n0 = (loc / gmn) * OBN;

  // Lane i of a load fetches row i >> 2 of its 16-row block, logical chunk lc.
  const int lc = (lane & 3) ^ ((lane >> 4) & 3);
  const __bf16 *A = (const __bf16 *)p.a;
  int64_t a_off[LA];
  const __bf16 *bp[LB];
#pragma unroll
  for (int q = 0; q < LA; ++q)
    a_off[q] = (int64_t)min(m0 + 16 * (wave * LA + q) + (lane >> 2), p.M - 1) * p.lda + 8 * lc;
#pragma unroll
  for (int q = 0; q < LB; ++q) {
    const int rb = 16 * (wave * LB + q) + (lane >> 2);   // staged B row
    if (GATED) {
      const int j = (rb % WTN) / 32;   // the wave's 32-row block: even gate, odd up
      const int col = n0 + (rb / WTN) * (WTN / 2) + (j >> 1) * 32 + rb % 32;
      bp[q] = (const __bf16 *)(j & 1 ? p.b2 : p.b) + (int64_t)min(col, p.N - 1) * p.b_sn + 8 * lc;
    } else {
      bp[q] = (const __bf16 *)p.b + (int64_t)min(n0 + rb, p.N - 1) * p.b_sn + 8 * lc;
    }
  }
  const int nk = (p.K + DBK - 1) / DBK;

  // Stage kt >= nk (issued so that every loop iteration has the same shape)
  // fetches valid data into a ring buffer nobody reads.
  auto issue = [&](int kt) {
    char *sb = lds + (kt & (DST - 1)) * STAGE;
    const int k0 = kt * DBK;
    // In the K tail a chunk past K fetches k = K - 8 of its row instead.
    const int kk = k0 + DBK <= p.K ? k0 : min(k0 + 8 * lc, p.K - 8) - 8 * lc;
#pragma unroll
    for (int q = 0; q < LA; ++q)
      __builtin_amdgcn_global_load_lds(A + a_off[q] + kk, sb + (wave * LA + q) * 1024, 16, 0, 0);
#pragma unroll
    for (int q = 0; q < LB; ++q)
      __builtin_amdgcn_global_load_lds(bp[q] + kk, sb + A_BYTES + (wave * LB + q) * 1024, 16, 0, 0);
  };
  // After stage kt (the K tail) has landed: zero the chunks past K.
  auto zero_tail = [&](int kt) {
    if (kt * DBK + 8 * lc >= p.K) {
      char *sb = lds + (kt & (DST - 1)) * STAGE + lane * 16;
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int q = 0; q < LA; ++q) *(u32x4 *)(sb + (wave * LA + q) * 1024) = z;
#pragma unroll
      for (int q = 0; q < LB; ++q) *(u32x4 *)(sb + A_BYTES + (wave * LB + q) * 1024) = z;
    }
  };
  // Wait until this wave's loads of stage s have landed (stages s+1 and s+2
  // may still be in flight), then zero the K tail if stage s holds it.
  auto wait_stage = [&](int s) {
    wait_vmcnt<2 * L>();
    if (s < nk && s * DBK + DBK > p.K) zero_tail(s);
  };

  struct Frags {
    bf16x8 a[4], b[NBW];
  };
  const int sx = (l32 >> 2) & 3;
  const int pc0 = (h2 ^ sx) * 16, pc1 = ((2 + h2) ^ sx) * 16;
  const int rowa = (wm * 128 + l32) * 64, rowb = A_BYTES + (wn * WTN + l32) * 64;
  auto frags = [&](int kt, int ks, Frags &f) {
    const char *sb = lds + (kt & (DST - 1)) * STAGE + (ks ? pc1 : pc0);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = *(const bf16x8 *)(sb + rowa + i * 2048);
#pragma unroll
    for (int j = 0; j < NBW; ++j) f.b[j] = *(const bf16x8 *)(sb + rowb + j * 2048);
  };

  f32x16 acc[4][NBW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = f32x16{};
  auto mfmas = [&](const Frags &f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  };

  // One iteration: [issue stage kt+3 | read fragments of k-step 1 | MFMAs of
  // k-step 0] interleaved one MFMA to one memory instruction, then wait for
  // stage kt+1 and barrier, then [read k-step 0 of stage kt+1 | MFMAs of
  // k-step 1], again interleaved.  With one wave per SIMD nothing else can
  // issue MFMAs while a wave issues loads, so they go between its MFMAs.
  Frags f0, f1;
  if (nk > 0) {
#pragma unroll
    for (int s = 0; s < DST - 1; ++s) issue(s);
    wait_stage(0);
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    frags(0, 0, f0);
    for (int kt = 0; kt < nk; ++kt) {
      // f0, read after the previous barrier, has had a block of MFMAs to land;
      // waiting for it here keeps the compiler from waiting on f1 below.
      wait_lgkmcnt0();
      __builtin_amdgcn_sched_barrier(0);
      // Stage kt+3 reuses the buffer of stage kt-1, whose last reads finished
      // before the previous barrier.
      issue(kt + DST - 1);
      frags(kt, 1, f1);
      mfmas(f0);
#pragma unroll
      for (int i = 0; i < L; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load (to LDS)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * NBW - L, 0);
      __builtin_amdgcn_sched_barrier(0);
      wait_stage(kt + 1);
      wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      frags(kt + 1, 0, f0);   // past the last stage: an unused read of a ring buffer
      mfmas(f1);
#pragma unroll
      for (int i = 0; i < L; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * NBW - L, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();   // no LDS-bound load may outlive the workgroup
  }

  auto store4 = [&](int gm, int gn, const f32x4 &v) {
    const int64_t off = (int64_t)gm * p.ldc + gn;
    if (p.c_f32) {
      float *c = (float *)p.c + off;
      if (p.c_vec) *(f32x4 *)c = v;
      else c[0] = v[0], c[1] = v[1], c[2] = v[2], c[3] = v[3];
    } else {
      __bf16 *c = (__bf16 *)p.c + off;
      const bf16x4 w = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
      if (p.c_vec) *(bf16x4 *)c = w;
      else c[0] = w[0], c[1] = w[1], c[2] = w[2], c[3] = w[3];
    }
  };
  auto store_all = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int gm = m0 + wm * 128 + i * 32 + l32;
      if (gm >= p.M) continue;
      if constexpr (GATED) {
#pragma unroll
        for (int u = 0; u < NBW / 2; ++u)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int gn = n0 + wn * (WTN / 2) + u * 32 + 8 * r4 + 4 * h2;
            if (gn >= p.N) continue;
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = activate(acc[i][2 * u][4 * r4 + e], ACT) * acc[i][2 * u + 1][4 * r4 + e];
            store4(gm, gn, v);
          }
      } else {
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int gn = n0 + wn * WTN + j * 32 + 8 * r4 + 4 * h2;
            if (gn >= p.N) continue;
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = activate(acc[i][j][4 * r4 + e], ACT);
            store4(gm, gn, v);
          }
      }
    }
  };
  store_all();
}

// One plain kernel per tile width (the body is a template).
#define CHAIN_DTL_KERNEL(NAME, NBW, GATED, ACT)                                            \
  __global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) \
  void NAME(const GemmParams p) { gemm_bf16_dtl<NBW, GATED, ACT>(p); }
#define CHAIN_DTL_KERNELS(SUFFIX, ACT)                                             \
  CHAIN_DTL_KERNEL(gemm_bf16_dtl_kernel_2_##SUFFIX, 2, false, ACT)                 \
  CHAIN_DTL_KERNEL(gemm_bf16_dtl_kernel_3_##SUFFIX, 3, false, ACT)                 \
  CHAIN_DTL_KERNEL(gemm_bf16_dtl_kernel_4_##SUFFIX, 4, false, ACT)                 \
  CHAIN_DTL_KERNEL(gemm_bf16_dtl_gated_kernel_2_##SUFFIX, 2, true, ACT)            \
  CHAIN_DTL_KERNEL(gemm_bf16_dtl_gated_kernel_4_##SUFFIX, 4, true, ACT)
CHAIN_DTL_KERNELS(erf, CHAIN_ACT_GELU_ERF)
CHAIN_DTL_KERNELS(tanh, CHAIN_ACT_GELU_TANH)
CHAIN_DTL_KERNELS(id, CHAIN_ACT_IDENTITY)
CHAIN_DTL_KERNELS(silu, CHAIN_ACT_SILU)
#undef CHAIN_DTL_KERNELS
#undef CHAIN_DTL_KERNEL

// Eight-wave kernel of the gated k-contiguous path (two waves per SIMD): a
// 256 x BN tile as 4 x 2 waves of 64 x BN/2, each a 2 x NBW grid of 32 x 32
// blocks with f32 accumulators in registers.  The ring, the stage depth, the swizzle and
// the k order are those of gemm_bf16_dtl (so both give the same bits); the
// loads are buffer loads that write LDS directly, addressed by a descriptor
// over the tile's rows (32-bit offsets: the host picks this kernel only when
// a tile's rows span less than 2^31 bytes), with the stage's k offset in the
// scalar offset operand.  A second wave on each SIMD issues MFMAs while the
// other waits on its fragment reads or the barrier.
//
// BKM false (gated only) takes the gate and up weights row-major ([K, N], n
// contiguous, one row stride): a stage's B block is then two row-major 32 x OBN
// sub-blocks, gate then up, each filled by whole 1 KB loads (so every load
// reads through one descriptor) with 64-byte groups XOR-swizzled by row as in
// gemm_bf16_w8r, and read with ds_read_b64_tr_b16.
template <int NBW, bool GATED, int ACT, bool BKM = true, int SD = DBK>
__device__ __forceinline__ void gemm_bf16_w8(const GemmParams &p) {
  constexpr int BN = 64 * NBW, WTN = 32 * NBW;
  constexpr int OBN = GATED ? BN / 2 : BN;   // output columns per tile
  static_assert(!GATED || NBW % 2 == 0, "gated tiles pair 32-row blocks");
  // SD: k per stage, 32 (a ring of four stages) or 64 (two), as in gemm_bf16_w8r
  static_assert(SD == 32 || SD == 64, "stage depth");
  constexpr int NS = SD == 32 ? 4 : 2, KST = SD / 16;
  constexpr int CPR = SD / 8, RPL = 64 / CPR, RBY = 2 * SD;
  auto kswz = [](int r) { return SD == 32 ? ((r >> 2) & 3) : ((r >> 1) & 7); };
  constexpr int A_BYTES = BM * SD * 2, B_BYTES = BN * SD * 2, STAGE = A_BYTES + B_BYTES;
  static_assert(NS * STAGE <= 160 * 1024, "the ring must fit in LDS");
  constexpr int NLB = B_BYTES / 1024;           // 1 KB loads of B per stage
  constexpr int LA = A_BYTES / 1024 / 8;        // 1 KB loads of A per wave and stage
  constexpr int LBH = (NLB + 7) / 8, LBL = NLB / 8;   // of B: waves below NLB % 8 take LBH
  static_assert(BKM || GATED, "row-major B: gated tiles only (a load never spans the two sub-blocks)");
  constexpr int BCH = OBN / 8, BG = OBN / 32;   // row-major sub-block: 16-byte chunks, 64-byte groups per row
  constexpr int SUB = SD * OBN * 2;             // bytes of a row-major sub-block
  auto row_swz = [](int r) { return BG % 4 == 0 ? (r & 3) : BG % 4 == 2 ? ((r >> 1) & 1) : 0; };
  __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  const bool hi = LBH == LBL || wave < NLB % 8;   // this wave takes LBH loads of B

  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + OBN - 1) / OBN;
  const int t = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  constexpr int GM = 4;
  const int g = t / (GM * tiles_n), fm = g * GM;
  const int gmn = min(GM, tiles_m - fm), loc = t - g * GM * tiles_n;
  const int m0 = (fm + loc % gmn) * BM, n0 = (loc / gmn) * OBN;

  // Descriptors over the tile's rows of A and of B (k contiguous in both; gated:
  // one over the gate rows and one over the up rows of the tile's columns).
  const int ra = min(p.M - m0, BM), rb = min(p.N - n0, OBN);
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const __bf16 *)p.a + (int64_t)m0 * p.lda), 0,
      (int)(((int64_t)(ra - 1) * p.lda + p.K) * 2), 0x00020000);
  const int64_t bspan = BKM ? (int64_t)(rb - 1) * p.b_sn + p.K : (int64_t)(p.K - 1) * p.b_sk + rb;
  const int64_t bbase = BKM ? (int64_t)n0 * p.b_sn : n0;
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const __bf16 *)p.b + bbase), 0, (int)(bspan * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t brs2 = GATED ? __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const __bf16 *)p.b2 + bbase), 0, (int)(bspan * 2), 0x00020000) : brs;
  // Staged B row r holds output column n0 + bcol(r) of B, or (gated) of B2 when
  // bup(r): each wave's 32-row blocks alternate gate, up for the same 32 columns.
  auto bcol = [](int r) {
    if (!GATED) return r;
    return (r / WTN) * (WTN / 2) + ((r % WTN) / 32 >> 1) * 32 + r % 32;
  };
  auto bup = [](int r) { return GATED && (((r % WTN) / 32) & 1); };
  // Lane i of a k-major load fetches row i / CPR of its RPL-row group, logical
  // chunk lc (the swizzle depends on the group only through the wave's parity).
  const int lc = (lane % CPR) ^ kswz(RPL * wave + lane / CPR);
  uint32_t aoff[LA], boff[LBH];
#pragma unroll
  for (int q = 0; q < LA; ++q)
    aoff[q] = (uint32_t)min(RPL * (wave + 8 * q) + lane / CPR, ra - 1) * (uint32_t)p.lda * 2u + 16u * lc;
  // Row-major: load L = wave + 8 q fills sub-block L / (NLB / 2) (gate, up);
  // its lane takes chunk g of the sub-block, row brow(q), columns bcolr(q) ..+7
  // (past the tile's last column: its last chunk again).
  auto bsub = [&](int q) { return (wave + 8 * q) / (NLB / 2); };
  auto brow = [&](int q) { return (64 * ((wave + 8 * q) % (NLB / 2)) + lane) / BCH; };
  auto bcolr = [&](int q) {
    const int c = (64 * ((wave + 8 * q) % (NLB / 2)) + lane) % BCH;
    return min(8 * (4 * ((c >> 2) ^ row_swz(brow(q))) + (c & 3)), rb - 8);
  };
#pragma unroll
  for (int q = 0; q < LBH; ++q)
    boff[q] = BKM ? (uint32_t)min(bcol(RPL * (wave + 8 * q) + lane / CPR), rb - 1) * (uint32_t)p.b_sn * 2u + 16u * lc
                  : (uint32_t)brow(q) * (uint32_t)p.b_sk * 2u + 2u * (uint32_t)bcolr(q);
  // the descriptor of load q: k-major, by its staged rows; row-major, by its sub-block
  auto bdesc = [&](int q) { return (BKM ? bup(RPL * (wave + 8 * q)) : bsub(q) == 1) ? brs2 : brs; };
  const int nk = (p.K + SD - 1) / SD;
  typedef __attribute__((address_space(3))) void lds_void;

  // Stage kt into ring slot kt % NS; past the last stage, stage 0 again (valid
  // data into a slot nobody reads, so every iteration has the same shape).
  auto issue = [&](int kt, auto whole_c) {
    char *sb = lds + (kt & (NS - 1)) * STAGE;
    const int k0 = kt < nk ? kt * SD : 0;
    if (decltype(whole_c)::value || k0 + SD <= p.K) {
#pragma unroll
      for (int q = 0; q < LA; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void *)(sb + (wave + 8 * q) * 1024), 16, aoff[q],
                                                 2 * k0, 0, 0);
#pragma unroll
      for (int q = 0; q < LBH; ++q)
        if (q < LBL || hi)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              bdesc(q), (lds_void *)(sb + A_BYTES + (wave + 8 * q) * 1024), 16, boff[q],
              BKM ? 2 * k0 : (int)((uint32_t)k0 * (uint32_t)p.b_sk * 2u), 0, 0);
    } else if constexpr (!BKM) {
      // K tail: A chunks past K fetch k = K - 8 of their row, B rows past K row K - 1
      const uint32_t kb = 2u * (uint32_t)min(k0 + 8 * lc, p.K - 8) - 16u * lc;
#pragma unroll
      for (int q = 0; q < LA; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void *)(sb + (wave + 8 * q) * 1024), 16, aoff[q] + kb,
                                                 0, 0, 0);
#pragma unroll
      for (int q = 0; q < LBH; ++q)
        if (q < LBL || hi) {
          const uint32_t r = (uint32_t)min(k0 + brow(q), p.K - 1);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(bdesc(q), (lds_void *)(sb + A_BYTES + (wave + 8 * q) * 1024), 16,
                                                   r * (uint32_t)p.b_sk * 2u + 2u * (uint32_t)bcolr(q), 0, 0, 0);
        }
    } else {
      // K tail: a chunk past K fetches k = K - 8 of its row instead
      const uint32_t kb = 2u * (uint32_t)min(k0 + 8 * lc, p.K - 8) - 16u * lc;
#pragma unroll
      for (int q = 0; q < LA; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void *)(sb + (wave + 8 * q) * 1024), 16, aoff[q] + kb,
                                                 0, 0, 0);
#pragma unroll
      for (int q = 0; q < LBH; ++q)
        if (q < LBL || hi)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(bup(RPL * (wave + 8 * q)) ? brs2 : brs,
                                                   (lds_void *)(sb + A_BYTES + (wave + 8 * q) * 1024), 16,
                                                   boff[q] + kb, 0, 0, 0);
    }
  };
  // After stage kt (the K tail) has landed: zero the chunks past K.
  auto zero_tail = [&](int kt) {
    char *sb = lds + (kt & (NS - 1)) * STAGE + lane * 16;
    const u32x4 z = {0u, 0u, 0u, 0u};
    if (kt * SD + 8 * lc >= p.K) {
#pragma unroll
      for (int q = 0; q < LA; ++q) *(u32x4 *)(sb + (wave + 8 * q) * 1024) = z;
      if constexpr (BKM) {
#pragma unroll
        for (int q = 0; q < LBH; ++q)
          if (q < LBL || hi) *(u32x4 *)(sb + A_BYTES + (wave + 8 * q) * 1024) = z;
      }
    }
    if constexpr (!BKM) {
#pragma unroll
      for (int q = 0; q < LBH; ++q)
        if ((q < LBL || hi) && kt * SD + brow(q) >= p.K) *(u32x4 *)(sb + A_BYTES + (wave + 8 * q) * 1024) = z;
    }
  };
  // This wave's loads of stage s have landed (the NS - 2 stages after it may
  // still be in flight); zero the K tail if stage s holds it.
  auto wait_landed = [&]() {
    if (hi) wait_vmcnt<(NS - 2) * (LA + LBH)>();
    else wait_vmcnt<(NS - 2) * (LA + LBL)>();
  };
  auto wait_stage = [&](int s) {
    wait_landed();
    if (s < nk && s * SD + SD > p.K) zero_tail(s);
  };

  struct Frags {
    bf16x8 a[2], b[NBW];
  };
  int pc[KST];
#pragma unroll
  for (int ks = 0; ks < KST; ++ks) pc[ks] = ((2 * ks + h2) ^ kswz(l32)) * 16;
  const int rowa = (wm * 64 + l32) * RBY, rowb = A_BYTES + (wn * WTN + l32) * RBY;
  // row-major: the transposing-read address of block j (gate for even j, up
  // for odd, output column block wn NBW / 2 + j / 2): k row 8 h2 + (lane & 15) / 4
  int trb[NBW];
  if constexpr (!BKM) {
    const int tr = (lane & 15) >> 2;
#pragma unroll
    for (int j = 0; j < NBW; ++j)
      trb[j] = A_BYTES + (j & 1) * SUB + (8 * h2 + tr) * 2 * OBN + ((wn * (NBW / 2) + (j >> 1)) ^ row_swz(tr)) * 64 +
               2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  }
  auto frags = [&](int kt, int ks, Frags &f) {
    const char *sb = lds + (kt & (NS - 1)) * STAGE + pc[ks];
#pragma unroll
    for (int i = 0; i < 2; ++i) f.a[i] = *(const bf16x8 *)(sb + rowa + i * 32 * RBY);
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      if constexpr (BKM) {
        f.b[j] = *(const bf16x8 *)(sb + rowb + j * 32 * RBY);
      } else {   // k rows 16 ks + 8 h2 + 0..3, then + 4..7
        const __bf16 *src = (const __bf16 *)(lds + (kt & (NS - 1)) * STAGE + trb[j] + ks * 16 * 2 * OBN);
        const i16x4 lo = ds_read_tr(src), hi4 = ds_read_tr(src + 4 * OBN);
        f.b[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };

  f32x16 acc[2][NBW];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = f32x16{};
  auto mfmas = [&](const Frags &f) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  };

  constexpr int NM = 2 * NBW;   // MFMAs per k-step
  Frags f0, f1;
  // The main loop, with the loads of stage kt+NS-1 spread one per MFMA of the
  // first k-step; each k-step's MFMAs run while the next k-step's fragments
  // are read (f0 and f1 alternate).  With K a multiple of the stage depth (the
  // usual case) no stage has a K tail and the loads take the branch-free path.
  auto run = [&](auto whole_c) {
    constexpr bool WHOLE = decltype(whole_c)::value;
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s, whole_c);
    wait_stage(0);
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    frags(0, 0, f0);
    for (int kt = 0; kt < nk; ++kt) {
      wait_lgkmcnt0();
      __builtin_amdgcn_sched_barrier(0);
      // stage kt+NS-1 reuses the slot of stage kt-1, whose reads all came
      // before the previous barrier
      issue(kt + NS - 1, whole_c);
      frags(kt, 1, f1);
      mfmas(f0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // load to LDS
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (KST == 4) {   // k-steps 1 and 2 (k-step 3 closes the stage below)
        frags(kt, 2, f0);
        mfmas(f1);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        frags(kt, 3, f1);
        mfmas(f0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 3);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (WHOLE) {
        wait_landed();
      } else {
        wait_stage(kt + 1);
      }
      wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      frags(kt + 1, 0, f0);   // past the last stage: an unused read of a ring slot
      mfmas(f1);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();   // no LDS-bound load may outlive the workgroup
  };
  if (nk > 0) {
    if (p.K % SD == 0) run(std::true_type{});
    else run(std::false_type{});
  }

  gemm_store_tile<2, NBW, GATED, ACT>(p, acc, m0 + wm * 64, n0 + wn * (GATED ? WTN / 2 : WTN), l32, h2);
}

// The 128-output-column gated tiles (256 staged B rows) take 64-deep stages,
// the 64-column ones 32-deep (too few MFMAs per stage to hide a two-stage ring).
#define CHAIN_W8_KERNEL(NAME, NBW, GATED, ACT, BKM, SD)                                       \
  __global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2))) \
  void NAME(const GemmParams p) { gemm_bf16_w8<NBW, GATED, ACT, BKM, SD>(p); }
#define CHAIN_W8_KERNELS(SUFFIX, ACT)                                             \
  CHAIN_W8_KERNEL(gemm_bf16_w8_gated_kernel_2_##SUFFIX, 2, true, ACT, true, 32)   \
  CHAIN_W8_KERNEL(gemm_bf16_w8_gated_kernel_4_##SUFFIX, 4, true, ACT, true, 64)   \
  CHAIN_W8_KERNEL(gemm_bf16_w8t_gated_kernel_2_##SUFFIX, 2, true, ACT, false, 32) \
  CHAIN_W8_KERNEL(gemm_bf16_w8t_gated_kernel_4_##SUFFIX, 4, true, ACT, false, 64)
CHAIN_W8_KERNELS(erf, CHAIN_ACT_GELU_ERF)
CHAIN_W8_KERNELS(tanh, CHAIN_ACT_GELU_TANH)
CHAIN_W8_KERNELS(id, CHAIN_ACT_IDENTITY)
CHAIN_W8_KERNELS(silu, CHAIN_ACT_SILU)
#undef CHAIN_W8_KERNELS
#undef CHAIN_W8_KERNEL

// Eight-wave kernel of the non-gated k-contiguous path: a 256 x 32 (NB0 + NB1)
// tile as 4 x 2 waves of 64 rows; waves 0-3 take the first NB0 column blocks,
// waves 4-7 the other NB1 (NB0 = NB1 for 128-, 192- and 256-wide tiles).  The
// columns may split unevenly: waves w and w+4 share a SIMD, so every SIMD
// still issues the MFMAs of NB0 + NB1 blocks per k-step.  With
// NB0 = 6, NB1 = 5 (352 columns), N = 1376 is four tiles per 256 rows (2.3 %
// padding) and M = 16384 one round of 256 tiles, where 192-wide tiles pad by
// 11.6 % and take two rounds.  Six blocks of accumulators (192 registers) leave
// no room for a second fragment set, so fragments are streamed (at every width:
// it also beats a double-buffered k-step by about 1 % at 256): each is read
// PD MFMAs before its first use, and the stage's wait and barrier sit PD MFMAs
// before its end, after the last read of the stage and before the reads of the
// next.  The k order is that of the gated and four-wave kernels, so all give
// the same bits.
//
// Stage depth SD: 32 k in a ring of four stages (three in flight), or 64 k in
// a ring of two (one in flight).  With 64 a k-major row of a stage is 128
// bytes, so each row's request to the L2 is a whole 128-byte line where 32
// takes half a line per stage (and the other half again a stage later): about
// 30 % fewer L2 requests for the same bytes.  Two stages in flight less hide
// the load latency only where a stage has enough MFMAs, so 64 serves the 256-
// and 352-wide tiles and 32 the narrower ones.
//
// BKM false takes B row-major ([K, N], n contiguous): load q of a wave then
// covers 64 consecutive 16-byte chunks of the stage's SD x BN block in row
// order, and a B fragment is two ds_read_b64_tr_b16 of four k rows.  A
// transposing read takes 64 bytes (a 64-byte group) of each of four
// consecutive rows; the groups of row r are XOR-swizzled by row_swz(r) so that
// the four land on disjoint banks (at 352 columns the 704-byte pitch already
// does that).
template <int NB0, int NB1, int ACT, bool BKM = true, int SD = DBK>
__device__ __forceinline__ void gemm_bf16_w8r(const GemmParams &p) {
  constexpr int BN = 32 * (NB0 + NB1);
  // SD: k per stage, 32 (a ring of four stages) or 64 (two).  A k-major row
  // of a stage is SD / 8 16-byte chunks, RPL rows per 1 KB load; chunk c of
  // row r sits at c ^ kswz(r), so that the 16-byte fragment reads of 16
  // consecutive rows hit 16 distinct bank groups.
  static_assert(SD == 32 || SD == 64, "stage depth");
  constexpr int NS = SD == 32 ? 4 : 2;
  constexpr int CPR = SD / 8, RPL = 64 / CPR, RBY = 2 * SD;
  auto kswz = [](int r) { return SD == 32 ? ((r >> 2) & 3) : ((r >> 1) & 7); };
  constexpr int BCH = BN / 8, BG = BN / 32;     // 16-byte chunks, 64-byte groups per row-major B row
  // Pitch 64 BG bytes: rows r..r+3 start 16 BG banks apart.  BG = 0 mod 4: all
  // on one bank group, swizzle by r & 3; BG = 2 mod 4: two apart, by (r >> 1) & 1.
  auto row_swz = [](int r) { return BG % 4 == 0 ? (r & 3) : BG % 4 == 2 ? ((r >> 1) & 1) : 0; };
  constexpr int A_BYTES = BM * SD * 2, B_BYTES = BN * SD * 2, STAGE = A_BYTES + B_BYTES;
  static_assert(NS * STAGE <= 160 * 1024, "the ring must fit in LDS");
  constexpr int NLB = B_BYTES / 1024;           // 1 KB loads of B per stage
  constexpr int LA = A_BYTES / 1024 / 8;        // 1 KB loads of A per wave and stage
  constexpr int LBH = (NLB + 7) / 8, LBL = NLB / 8;   // of B: waves below NLB % 8 take LBH
  __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const int wm = wave & 3, wn = wave >> 2;
  const bool hi = LBH == LBL || wave < NLB % 8;   // this wave takes LBH loads of B

  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int t = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  constexpr int GM = 4;
  const int g = t / (GM * tiles_n), fm = g * GM;
  const int gmn = min(GM, tiles_m - fm), loc = t - g * GM * tiles_n;
  const int m0 = (fm + loc % gmn) * BM, n0 = (loc / gmn) * BN;

  const int ra = min(p.M - m0, BM), rb = min(p.N - n0, BN);
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const __bf16 *)p.a + (int64_t)m0 * p.lda), 0,
      (int)(((int64_t)(ra - 1) * p.lda + p.K) * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t brs =
      BKM ? __builtin_amdgcn_make_buffer_rsrc((void *)((const __bf16 *)p.b + (int64_t)n0 * p.b_sn), 0,
                                              (int)(((int64_t)(rb - 1) * p.b_sn + p.K) * 2), 0x00020000)
          : __builtin_amdgcn_make_buffer_rsrc((void *)((const __bf16 *)p.b + n0), 0,
                                              (int)(((int64_t)(p.K - 1) * p.b_sk + rb) * 2), 0x00020000);
  // Lane i of a k-major load fetches row i / CPR of its RPL-row group, logical
  // chunk lc; load q of a wave covers the group wave + 8 q of its operand (the
  // swizzle of those rows depends on the group only through the wave's parity).
  const int lc = (lane % CPR) ^ kswz(RPL * wave + lane / CPR);
  uint32_t aoff[LA], boff[LBH];
#pragma unroll
  for (int q = 0; q < LA; ++q)
    aoff[q] = (uint32_t)min(RPL * (wave + 8 * q) + lane / CPR, ra - 1) * (uint32_t)p.lda * 2u + 16u * lc;
  // Row-major B: chunk 64 (wave + 8 q) + lane of a stage is row brow(q), columns
  // bcol(q) .. + 7 (past the tile's last column: its last chunk again).
  auto brow = [&](int q) { return (64 * (wave + 8 * q) + lane) / BCH; };
  auto bcol = [&](int q) {
    const int c = (64 * (wave + 8 * q) + lane) % BCH;
    return min(8 * (4 * ((c >> 2) ^ row_swz(brow(q))) + (c & 3)), rb - 8);
  };
#pragma unroll
  for (int q = 0; q < LBH; ++q)
    boff[q] = BKM ? (uint32_t)min(RPL * (wave + 8 * q) + lane / CPR, rb - 1) * (uint32_t)p.b_sn * 2u + 16u * lc
                  : (uint32_t)brow(q) * (uint32_t)p.b_sk * 2u + 2u * (uint32_t)bcol(q);
  const int nk = (p.K + SD - 1) / SD;
  typedef __attribute__((address_space(3))) void lds_void;

  // Load q of this wave for stage kt (q < LA: A, else B) into ring slot kt % NS;
  // past the last stage, stage 0 again into a slot nobody reads.  Whole stages
  // carry the k offset in the scalar offset; in the K tail a chunk past K
  // fetches k = K - 8 of its row instead.
  auto issue_one = [&](int kt, int q, auto whole_c) {
    char *sb = lds + (kt & (NS - 1)) * STAGE;
    const int k0 = kt < nk ? kt * SD : 0;
    const bool whole = decltype(whole_c)::value || k0 + SD <= p.K;
    const uint32_t kv = whole ? 0u : 2u * (uint32_t)min(k0 + 8 * lc, p.K - 8) - 16u * lc;
    const int ks = whole ? 2 * k0 : 0;
    if (q < LA) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void *)(sb + (wave + 8 * q) * 1024), 16, aoff[q] + kv,
                                               ks, 0, 0);
    } else if (q - LA < LBL || hi) {
      lds_void *dst = (lds_void *)(sb + A_BYTES + (wave + 8 * (q - LA)) * 1024);
      if constexpr (BKM) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, dst, 16, boff[q - LA] + kv, ks, 0, 0);
      } else if (whole) {   // the stage's first row in the scalar offset
        __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, dst, 16, boff[q - LA],
                                                 (int)((uint32_t)k0 * (uint32_t)p.b_sk * 2u), 0, 0);
      } else {              // K tail: a row past K fetches row K - 1, zeroed once landed
        const uint32_t r = (uint32_t)min(k0 + brow(q - LA), p.K - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, dst, 16, r * (uint32_t)p.b_sk * 2u + 2u * (uint32_t)bcol(q - LA),
                                                 0, 0, 0);
      }
    }
  };
  auto zero_tail = [&](int kt) {   // after stage kt (the K tail) has landed
    char *sb = lds + (kt & (NS - 1)) * STAGE + lane * 16;
    const u32x4 z = {0u, 0u, 0u, 0u};
    if (kt * SD + 8 * lc >= p.K) {
#pragma unroll
      for (int q = 0; q < LA; ++q) *(u32x4 *)(sb + (wave + 8 * q) * 1024) = z;
      if constexpr (BKM) {
#pragma unroll
        for (int q = 0; q < LBH; ++q)
          if (q < LBL || hi) *(u32x4 *)(sb + A_BYTES + (wave + 8 * q) * 1024) = z;
      }
    }
    if constexpr (!BKM) {
#pragma unroll
      for (int q = 0; q < LBH; ++q)
        if ((q < LBL || hi) && kt * SD + brow(q) >= p.K) *(u32x4 *)(sb + A_BYTES + (wave + 8 * q) * 1024) = z;
    }
  };
  // this wave's loads of the oldest stage in flight have landed (the NS - 2
  // stages after it may still be in flight)
  auto wait_landed = [&]() {
    if (hi) wait_vmcnt<(NS - 2) * (LA + LBH)>();
    else wait_vmcnt<(NS - 2) * (LA + LBL)>();
  };

  constexpr int KST = SD / 16;   // MFMA k-steps per stage
  int pc[KST];
#pragma unroll
  for (int ks = 0; ks < KST; ++ks) pc[ks] = ((2 * ks + h2) ^ kswz(l32)) * 16;
  const int rowa = (wm * 64 + l32) * RBY;

  auto body = [&](auto nbw_c, int col0) {
    constexpr int NBW = decltype(nbw_c)::value;
    // MFMA m of a stage (m = 0 .. NM-1): k-step m / 2NBW, B block (m / 2) % NBW,
    // A block m % 2.  The A pair and B block 0 of a k-step are read for its
    // first MFMA, B block j for MFMA 2j.
    constexpr int NM = 2 * KST * NBW, PD = 4;
    static_assert(PD % 2 == 0 && PD <= 2 * NBW, "reads run ahead within one k-step");
    const int rowb = A_BYTES + (col0 + l32) * RBY;
    // row-major B: this lane's transposing-read address within a stage for
    // column block j: k row 8 h2 + (lane & 15) / 4, column col0 + 32 j +
    // 16 ((lane >> 4) & 1) + 4 (lane & 3), its 64-byte group swizzled
    int trb[NBW];
    {
      const int tr = (lane & 15) >> 2;
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        trb[j] = A_BYTES + (8 * h2 + tr) * 2 * BN + (((col0 >> 5) + j) ^ row_swz(tr)) * 64 +
                 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    }
    bf16x8 fa[KST][2], fb[KST][NBW];
    f32x16 acc[2][NBW];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) acc[i][j] = f32x16{};
    auto read_at = [&](const char *sb, int u) {   // the fragments first used at MFMA u
      const int ks = u / (2 * NBW), r = u % (2 * NBW);
      const char *b = sb + pc[ks];
      if (r == 0) {
        fa[ks][0] = *(const bf16x8 *)(b + rowa);
        fa[ks][1] = *(const bf16x8 *)(b + rowa + 32 * RBY);
      }
      if (r % 2 == 0) {
        if constexpr (BKM) {
          fb[ks][r / 2] = *(const bf16x8 *)(b + rowb + (r / 2) * 32 * RBY);
        } else {   // k rows 16 ks + 8 h2 + 0..3, then + 4..7, of column block r / 2
          const __bf16 *src = (const __bf16 *)(sb + trb[r / 2] + ks * 16 * 2 * BN);
          const i16x4 lo = ds_read_tr(src), hi4 = ds_read_tr(src + 4 * BN);
          fb[ks][r / 2] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    };
    auto run = [&](auto whole_c) {
      constexpr bool WHOLE = decltype(whole_c)::value;
#pragma unroll
      for (int s = 0; s < NS - 1; ++s)
#pragma unroll
        for (int q = 0; q < LA + LBH; ++q) issue_one(s, q, whole_c);
      wait_landed();
      if (!WHOLE && SD > p.K) zero_tail(0);
      wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int u = 0; u < PD; ++u) read_at(lds, u);
      for (int kt = 0; kt < nk; ++kt) {
        const char *cur = lds + (kt & (NS - 1)) * STAGE;
        const char *nxt = lds + ((kt + 1) & (NS - 1)) * STAGE;   // past the last stage: an unused slot
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          if (m == NM - PD) {
            // every read of this stage is issued: once they are back, stage
            // kt+1 has landed and all waves are here, its slot may be refilled
            wait_lgkmcnt0();
            wait_landed();
            if (!WHOLE && kt + 1 < nk && (kt + 1) * SD + SD > p.K) zero_tail(kt + 1);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
          }
          if (m + PD < NM) read_at(cur, m + PD);
          else read_at(nxt, m + PD - NM);
          // stage kt+NS-1 refills the slot of stage kt-1, released at its barrier
          if (m < LA + LBH) issue_one(kt + NS - 1, m, whole_c);
          const int ks = m / (2 * NBW), j = (m / 2) % NBW, i = m % 2;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][j], fa[ks][i], acc[i][j], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      wait_vmcnt<0>();   // no LDS-bound load may outlive the workgroup
    };
    if (nk > 0) {
      if (p.K % SD == 0) run(std::true_type{});
      else run(std::false_type{});
    }
    gemm_store_tile<2, NBW, false, ACT>(p, acc, m0 + wm * 64, n0 + col0, l32, h2);
  };
  if (wn == 0) body(std::integral_constant<int, NB0>{}, 0);
  else body(std::integral_constant<int, NB1>{}, 32 * NB0);
}

#define CHAIN_W8R_KERNEL(NAME, NB0, NB1, ACT, BKM)                                            \
  __global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2))) \
  void NAME(const GemmParams p) { gemm_bf16_w8r<NB0, NB1, ACT, BKM>(p); }
// 64 k per stage (two stages) at 256 columns, and at 352 for k-major B (at 352
// row-major B would spill); 32 k per stage (four stages) otherwise.
#define CHAIN_W8R64_KERNEL(NAME, NB0, NB1, ACT, BKM)                                          \
  __global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2))) \
  void NAME(const GemmParams p) { gemm_bf16_w8r<NB0, NB1, ACT, BKM, 64>(p); }
#define CHAIN_W8R_KERNELS(SUFFIX, ACT)                                   \
  CHAIN_W8R_KERNEL(gemm_bf16_w8r_kernel_4_##SUFFIX, 2, 2, ACT, true)     \
  CHAIN_W8R_KERNEL(gemm_bf16_w8r_kernel_6_##SUFFIX, 3, 3, ACT, true)     \
  CHAIN_W8R64_KERNEL(gemm_bf16_w8r_kernel_8_##SUFFIX, 4, 4, ACT, true)   \
  CHAIN_W8R64_KERNEL(gemm_bf16_w8r_kernel_11_##SUFFIX, 6, 5, ACT, true)  \
  CHAIN_W8R_KERNEL(gemm_bf16_w8rt_kernel_4_##SUFFIX, 2, 2, ACT, false)   \
  CHAIN_W8R_KERNEL(gemm_bf16_w8rt_kernel_6_##SUFFIX, 3, 3, ACT, false)   \
  CHAIN_W8R64_KERNEL(gemm_bf16_w8rt_kernel_8_##SUFFIX, 4, 4, ACT, false) \
  CHAIN_W8R_KERNEL(gemm_bf16_w8rt_kernel_11_##SUFFIX, 6, 5, ACT, false)
CHAIN_W8R_KERNELS(erf, CHAIN_ACT_GELU_ERF)
CHAIN_W8R_KERNELS(tanh, CHAIN_ACT_GELU_TANH)
CHAIN_W8R_KERNELS(id, CHAIN_ACT_IDENTITY)
CHAIN_W8R_KERNELS(silu, CHAIN_ACT_SILU)
#undef CHAIN_W8R_KERNELS
#undef CHAIN_W8R64_KERNEL
#undef CHAIN_W8R_KERNEL

// f32 inputs: 128 x 128 x 32 tiles on v_mfma_f32_32x32x2_f32 (A: lane holds
// A[m][k0 + h2], B: lane holds B[k0 + h2][n]); exact f32 products, f32
// accumulation.
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
      bs[r][c] = (k0 + r < p.K && n0 + c < p.N)
                     ? B[(int64_t)(k0 + r) * p.b_sk + (int64_t)(n0 + c) * p.b_sn]
                     : 0.f;
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

template <int NBW>
void launch_bf16(const GemmParams &p, hipStream_t stream) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + 64 * NBW - 1) / (64 * NBW));
  const dim3 grid(tiles), block(512);
  switch (p.act) {
    case CHAIN_ACT_GELU_ERF: hipLaunchKernelGGL((gemm_bf16_kernel<NBW, CHAIN_ACT_GELU_ERF>), grid, block, 0, stream, p); break;
    case CHAIN_ACT_GELU_TANH: hipLaunchKernelGGL((gemm_bf16_kernel<NBW, CHAIN_ACT_GELU_TANH>), grid, block, 0, stream, p); break;
    case CHAIN_ACT_SILU: hipLaunchKernelGGL((gemm_bf16_kernel<NBW, CHAIN_ACT_SILU>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((gemm_bf16_kernel<NBW, CHAIN_ACT_IDENTITY>), grid, block, 0, stream, p);
  }
}

void launch_bf16_width(const GemmParams &p, int nbw, hipStream_t stream) {
  if (nbw == 4) launch_bf16<4>(p, stream);
  else if (nbw == 3) launch_bf16<3>(p, stream);
  else launch_bf16<2>(p, stream);
}

// The eight- and four-wave kernels address a tile's rows with 32-bit byte offsets.
bool rows_fit32(const GemmParams &p, int obn) {
  const int64_t span_a = ((int64_t)(min(p.M, BM) - 1) * p.lda + p.K) * 2;
  const int64_t span_b = ((int64_t)(min(p.N, obn) - 1) * p.b_sn + p.K) * 2;
  return span_a < ((int64_t)1 << 31) && span_b < ((int64_t)1 << 31);
}
bool w8_fits(const GemmParams &p, int nbw, bool gated) { return rows_fit32(p, gated ? 32 * nbw : 64 * nbw); }

// Gated: 32 * nbw output columns per tile; nbw 4 unless 2 fills the chip's
// rounds with less work per CU.
void launch_dtl_gated(const GemmParams &p, int cus, hipStream_t stream) {
  const int tm = (p.M + BM - 1) / BM;
  auto cost = [&](int nbw) {
    const int64_t tiles = (int64_t)tm * ((p.N + 32 * nbw - 1) / (32 * nbw));
    return ((tiles + cus - 1) / cus) * nbw;
  };
  const int nbw = cost(2) < cost(4) ? 2 : 4;
  const int tiles = tm * ((p.N + 32 * nbw - 1) / (32 * nbw));
  typedef void (*Kern)(const GemmParams);
  if (p.b_sk != 1) {   // row-major gate and up weights (gemm_gated_rowmajor_ok holds)
    static const Kern t2[4] = {gemm_bf16_w8t_gated_kernel_2_erf, gemm_bf16_w8t_gated_kernel_2_tanh,
                               gemm_bf16_w8t_gated_kernel_2_id, gemm_bf16_w8t_gated_kernel_2_silu};
    static const Kern t4[4] = {gemm_bf16_w8t_gated_kernel_4_erf, gemm_bf16_w8t_gated_kernel_4_tanh,
                               gemm_bf16_w8t_gated_kernel_4_id, gemm_bf16_w8t_gated_kernel_4_silu};
    hipLaunchKernelGGL((nbw == 4 ? t4 : t2)[p.act], dim3(tiles), dim3(512), 0, stream, p);
    return;
  }
  if (w8_fits(p, nbw, true)) {
    static const Kern w2[4] = {gemm_bf16_w8_gated_kernel_2_erf, gemm_bf16_w8_gated_kernel_2_tanh,
                               gemm_bf16_w8_gated_kernel_2_id, gemm_bf16_w8_gated_kernel_2_silu};
    static const Kern w4[4] = {gemm_bf16_w8_gated_kernel_4_erf, gemm_bf16_w8_gated_kernel_4_tanh,
                               gemm_bf16_w8_gated_kernel_4_id, gemm_bf16_w8_gated_kernel_4_silu};
    hipLaunchKernelGGL((nbw == 4 ? w4 : w2)[p.act], dim3(tiles), dim3(512), 0, stream, p);
    return;
  }
  static const Kern k2[4] = {gemm_bf16_dtl_gated_kernel_2_erf, gemm_bf16_dtl_gated_kernel_2_tanh,
                             gemm_bf16_dtl_gated_kernel_2_id, gemm_bf16_dtl_gated_kernel_2_silu};
  static const Kern k4[4] = {gemm_bf16_dtl_gated_kernel_4_erf, gemm_bf16_dtl_gated_kernel_4_tanh,
                             gemm_bf16_dtl_gated_kernel_4_id, gemm_bf16_dtl_gated_kernel_4_silu};
  hipLaunchKernelGGL((nbw == 4 ? k4 : k2)[p.act], dim3(tiles), dim3(256), 0, stream, p);
}

void launch_dtl(const GemmParams &p, int nbw, hipStream_t stream) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + 64 * nbw - 1) / (64 * nbw));
  typedef void (*Kern)(const GemmParams);
  static const Kern ks[3][4] = {
      {gemm_bf16_dtl_kernel_2_erf, gemm_bf16_dtl_kernel_2_tanh, gemm_bf16_dtl_kernel_2_id, gemm_bf16_dtl_kernel_2_silu},
      {gemm_bf16_dtl_kernel_3_erf, gemm_bf16_dtl_kernel_3_tanh, gemm_bf16_dtl_kernel_3_id, gemm_bf16_dtl_kernel_3_silu},
      {gemm_bf16_dtl_kernel_4_erf, gemm_bf16_dtl_kernel_4_tanh, gemm_bf16_dtl_kernel_4_id, gemm_bf16_dtl_kernel_4_silu}};
  hipLaunchKernelGGL(ks[nbw - 2][p.act], dim3(tiles), dim3(256), 0, stream, p);
}

// Non-gated eight-wave tiles: nbw = 2, 3, 4 (128, 192, 256 columns, even wave
// columns) or 11 (352 columns, 6 + 5).
void launch_w8(const GemmParams &p, int nbw, hipStream_t stream) {
  const int width = nbw == 11 ? 352 : 64 * nbw;
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + width - 1) / width);
  typedef void (*Kern)(const GemmParams);
  static const Kern ks[4][4] = {
      {gemm_bf16_w8r_kernel_4_erf, gemm_bf16_w8r_kernel_4_tanh, gemm_bf16_w8r_kernel_4_id, gemm_bf16_w8r_kernel_4_silu},
      {gemm_bf16_w8r_kernel_6_erf, gemm_bf16_w8r_kernel_6_tanh, gemm_bf16_w8r_kernel_6_id, gemm_bf16_w8r_kernel_6_silu},
      {gemm_bf16_w8r_kernel_8_erf, gemm_bf16_w8r_kernel_8_tanh, gemm_bf16_w8r_kernel_8_id, gemm_bf16_w8r_kernel_8_silu},
      {gemm_bf16_w8r_kernel_11_erf, gemm_bf16_w8r_kernel_11_tanh, gemm_bf16_w8r_kernel_11_id,
       gemm_bf16_w8r_kernel_11_silu}};
  hipLaunchKernelGGL(ks[nbw == 11 ? 3 : nbw - 2][p.act], dim3(tiles), dim3(512), 0, stream, p);
}

// Row-major B (n contiguous) on the eight-wave kernel: B's rows and base
// 16-byte aligned, N a multiple of 8, and B's column band of the widest tile
// within 32-bit byte offsets.
bool w8rt_fits(const GemmParams &p) {
  const int64_t span_a = ((int64_t)(min(p.M, BM) - 1) * p.lda + p.K) * 2;
  const int64_t span_b = ((int64_t)(p.K - 1) * p.b_sk + min(p.N, 352)) * 2;
  return p.b_sn == 1 && (uintptr_t)p.b % 16 == 0 && p.b_sk % 8 == 0 && p.N % 8 == 0 &&
         span_a < ((int64_t)1 << 31) && span_b < ((int64_t)1 << 31);
}
void launch_w8rt(const GemmParams &p, int nbw, hipStream_t stream) {
  const int width = nbw == 11 ? 352 : 64 * nbw;
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + width - 1) / width);
  typedef void (*Kern)(const GemmParams);
  static const Kern ks[4][4] = {
      {gemm_bf16_w8rt_kernel_4_erf, gemm_bf16_w8rt_kernel_4_tanh, gemm_bf16_w8rt_kernel_4_id,
       gemm_bf16_w8rt_kernel_4_silu},
      {gemm_bf16_w8rt_kernel_6_erf, gemm_bf16_w8rt_kernel_6_tanh, gemm_bf16_w8rt_kernel_6_id,
       gemm_bf16_w8rt_kernel_6_silu},
      {gemm_bf16_w8rt_kernel_8_erf, gemm_bf16_w8rt_kernel_8_tanh, gemm_bf16_w8rt_kernel_8_id,
       gemm_bf16_w8rt_kernel_8_silu},
      {gemm_bf16_w8rt_kernel_11_erf, gemm_bf16_w8rt_kernel_11_tanh, gemm_bf16_w8rt_kernel_11_id,
       gemm_bf16_w8rt_kernel_11_silu}};
  hipLaunchKernelGGL(ks[nbw == 11 ? 3 : nbw - 2][p.act], dim3(tiles), dim3(512), 0, stream, p);
}

int compute_units() {
  static thread_local int dev_cached = -1, cus = 256;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return cus;
  if (dev != dev_cached) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) cus = n;
    dev_cached = dev;
  }
  return cus;
}

}  // namespace

// Tile width for the bf16 path: the one that minimises rounds x (tile width +
// 64), one workgroup per CU; the time of a round grows with the tile width,
// plus a part that does not (its first stage loads and its output stores, about
// what 64 columns of MFMAs take at the FFN shard's shapes).  Eight-wave tiles
// are 64 x nbw wide (nbw 4, 3, 2); with wide = true the 352-wide tiles of the
// uneven split are a candidate too.  Returns nbw, or 11 for 352 columns.
int gemm_bf16_block_cols(int M, int N, int cus, bool wide) {
  int best = 4;
  int64_t best_cost = INT64_MAX;
  const int64_t tm = (M + BM - 1) / BM;
  auto cost = [&](int width) {
    const int64_t tiles = tm * ((N + width - 1) / width);
    return ((tiles + cus - 1) / cus) * (width + 64);
  };
  for (int nbw = 4; nbw >= 2; --nbw)
    if (cost(64 * nbw) < best_cost) best = nbw, best_cost = cost(64 * nbw);
  if (wide && cost(352) < best_cost) best = 11;
  return best;
}

bool gemm_gated_rowmajor_ok(const GemmParams &p) {
  const int64_t span_a = ((int64_t)(min(p.M, BM) - 1) * p.lda + p.K) * 2;
  const int64_t span_b = ((int64_t)(p.K - 1) * p.b_sk + min(p.N, 128)) * 2;
  return p.b_sn == 1 && (uintptr_t)p.b % 16 == 0 && (uintptr_t)p.b2 % 16 == 0 && p.b_sk % 8 == 0 &&
         p.N % 8 == 0 && span_a < ((int64_t)1 << 31) && span_b < ((int64_t)1 << 31);
}

hipError_t launch_gemm(const GemmParams &p, int dtype, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (p.gated) {
    if (dtype != CHAIN_BF16 || (p.b_sk != 1 && !gemm_gated_rowmajor_ok(p))) return hipErrorInvalidValue;
    launch_dtl_gated(p, compute_units(), stream);
  } else if (dtype == CHAIN_BF16) {
    const bool k_contig = p.b_sk == 1, rt = !k_contig && w8rt_fits(p);
    const int choice = gemm_bf16_block_cols(p.M, p.N, compute_units(), k_contig || rt);
    const int nbw = choice == 11 ? 4 : choice;
    if (k_contig) {
      if (rows_fit32(p, choice == 11 ? 352 : 64 * nbw)) launch_w8(p, choice, stream);
      else launch_dtl(p, nbw, stream);
    } else if (rt) {
      launch_w8rt(p, choice, stream);
    } else {
      launch_bf16_width(p, nbw, stream);
    }
  } else {
    const int tiles = ((p.M + TM - 1) / TM) * ((p.N + TN - 1) / TN);
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(tiles), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace chain
