// Attention backward on bf16 MFMA tiles (gfx950): dQ, dK, dV of
// O = softmax(scale * Q.K^T + causal mask).V, given O, its log-sum-exp and dO.
//
// The chain O = f(A.B).C is the core unit of Transformer training (METP
// article, abstract); its backward recomputes the probabilities from the
// saved log-sum-exp instead of storing them (2D-Attention summary, "Estrategias
// de Entrenamiento Distribuido": keep what is needed, recompute the rest).
// With P_ij = exp(s_ij - LSE_i) on the visible keys:
//   D_i = sum_d dO_id O_id,  dS = P * (dO.V^T - D),
//   dQ = scale * dS.K,  dK = scale * dS^T.Q,  dV = P^T.dO,
// dK and dV summed over the query heads that share a key/value head (GQA).
//
// Two kernels, no atomics (every output element is written once, so reruns
// give identical bits).  The scores are formed in base 2 from bf16 operands
// scaled by scale * log2(e) (Q in dq, as in the forward; K in dkdv); each S
// accumulator starts from -LSE * log2(e) (-inf where masked) and each dP
// accumulator of dkdv from -D, so P is one exp2 and dS one product.
//  - dq: eight waves (two per SIMD) take 32-row query blocks of WH heads of one
//    key/value head and walk the visible 64-key tiles.  Each wave first forms
//    D_i = sum_d dO_id O_id for its rows and writes -LSE_i * log2(e) and -D_i
//    to the workspace, in blocks of 16 rows [16 x -LSE*log2e | 16 x -D], rows
//    padded to a multiple of 64 with (-inf, 0) so that padding rows get
//    probability 0.  Per tile and wave:
//    S^T = K.Q^T and dP^T = V.dO^T (Q and dO fragments stay in registers, each
//    lane owns one query), dS^T = P^T * (dP^T - D) in registers, then
//    dQ^T += K^T.dS^T with K^T read by ds_read_b64_tr_b16 in the key order the
//    dS^T accumulator holds.
//  - dkdv (launched after dq, whose workspace rows it reads): four waves (one
//    per SIMD, for the two 32-key accumulators) take 128 keys of one key/value
//    head, 32 per wave with their K and V fragments in registers, and walk every
//    visible 64-row query tile of every query head of the group.  Per tile and wave, for its two 32-query halves: S = Q.K^T and
//    dP = dO.V^T, P and dS, then dV^T += dO^T.P and dK^T += Q^T.dS with dO^T
//    and Q^T read transposed.  With one wave per SIMD nothing else hides the
//    softmax, so the wave interleaves it by hand: the second half's S/dP MFMAs
//    carry the first half's softmax between them, and the first half's dV/dK
//    MFMAs the second half's.
// Tiles reach LDS by buffer loads that write LDS directly, into a ring of four
// stages fetched three tiles ahead, one barrier per tile.  A staged row's
// 16-byte chunks are XOR-swizzled so that both the 16-byte row-fragment reads
// and the transposing reads of the same tile hit distinct bank groups.  Query
// tiles (dq) and key blocks (dkdv) are taken in pairs t, T-1-t so causal work
// per workgroup is even, and workgroups of one key/value head share an XCD.
#include "internal.h"

namespace chain {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kAhead = 4;    // LDS fragments in flight ahead of their MFMA
constexpr int kRowPad = 64;  // workspace rows per head are padded to this multiple

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: in each group of 16 lanes, lane i receives element i%4
// of the 4-element rows addressed by lanes 4e + i/4, e = 0..3.  The restrict
// qualifier tells the compiler the read does not alias the direct-to-LDS loads
// in flight; without it, it waits for all of them (vmcnt(0)) before the read,
// which empties the three-tile prefetch ring at every key block.
__device__ inline i16x4 ds_read_tr(const char *__restrict__ p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Chunk swizzle of a staged tile row r (16-byte chunks, D/8 per row).  Bits 2-3
// of the D=128 form differ over any 4 aligned rows (the rows one transposing
// read touches per 32 lanes, over 4 consecutive chunks), and the whole form is
// a bijection over 16 consecutive rows (the rows 16 lanes of a 16-byte
// fragment read touch, all at one chunk).  For D=64 two rows share a 256-byte
// bank window, so the same holds with r/2 in place of r.
template <int D>
__device__ inline int swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// N MFMAs whose A operands are 16-byte LDS reads at addr(i), each read kAhead
// MFMAs before its use; op(i, a) issues MFMA i.
template <int N, typename Addr, typename Op>
__device__ __forceinline__ void run_b128(Addr addr, Op op) {
  constexpr int A = N < kAhead ? N : kAhead;
  bf16x8 f[A];
#pragma unroll
  for (int i = 0; i < A; ++i) f[i] = *(const bf16x8 *)addr(i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bf16x8 a = f[i % A];
    if (i + A < N) f[i % A] = *(const bf16x8 *)addr(i + A);
    op(i, a);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// N MFMAs whose A operands come from two transposing reads each, at lo(i) and
// hi(i) (k rows r..r+3 / r+8..r+11 of the lane's 16-row group).
template <int N, typename Lo, typename Hi, typename Op>
__device__ __forceinline__ void run_tr(Lo lo, Hi hi, Op op) {
  constexpr int A = N < kAhead ? N : kAhead;
  i16x4 fl[A], fh[A];
#pragma unroll
  for (int i = 0; i < A; ++i) {
    fl[i] = ds_read_tr(lo(i));
    fh[i] = ds_read_tr(hi(i));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const i16x8 a = __builtin_shufflevector(fl[i % A], fh[i % A], 0, 1, 2, 3, 4, 5, 6, 7);
    if (i + A < N) {
      fl[i % A] = ds_read_tr(lo(i + A));
      fh[i % A] = ds_read_tr(hi(i + A));
    }
    op(i, __builtin_bit_cast(bf16x8, a));
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Per-lane LDS byte offsets of the fragments of a staged tile with row pitch
// 2D bytes: aoff[ks] for the 16-byte row fragment of k-step ks (row l32, chunk
// 2ks + h2), tlo/thi[db] for the transposing reads of column block db (rows
// trow and trow + 8 of a 16-row-aligned group).
template <int D>
struct FragOffsets {
  static constexpr int KS = D / 16, DB = D / 32, RB = 2 * D;
  int aoff[KS], tlo[DB], thi[DB];
  __device__ __forceinline__ explicit FragOffsets(int lane) {
    const int h2 = lane >> 5, l32 = lane & 31;
    const int xa = swz<D>(l32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) aoff[ks] = l32 * RB + (((2 * ks + h2) ^ xa) << 4);
    const int trow = 4 * h2 + ((lane & 15) >> 2);
    const int ylane = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      tlo[db] = trow * RB + (((4 * db + ylane) ^ swz<D>(trow)) << 4) + 8 * (lane & 1);
      thi[db] = (trow + 8) * RB + (((4 * db + ylane) ^ swz<D>(trow + 8)) << 4) + 8 * (lane & 1);
    }
  }
};

__device__ inline int padded_rows(int S) { return (S + kRowPad - 1) / kRowPad * kRowPad; }

// Float index of row r's -LSE*log2e in its head's workspace block; -D_i is 16 further.
__device__ inline int rv_index(int r) { return (r >> 4) * 32 + (r & 15); }

// ---- dQ ----------------------------------------------------------------------
template <int D, int WH>
__device__ __forceinline__ void dq_body(const AttnBwdParams &p) {
  constexpr int NW = 8, WQ = NW / WH, ROWS = 32 * WQ, BN = 64;
  constexpr int KS = D / 16, DB = D / 32, RB = 2 * D, CPR = D / 8, RPL = 64 / CPR;
  constexpr int TB = BN * RB;            // bytes of one staged K or V tile
  constexpr int SB = 2 * TB;             // a stage: K tile, then V tile
  constexpr int NST = 4;
  constexpr int LPW = BN / RPL / NW;     // 1 KB loads per wave and operand
  constexpr int LT = 2 * LPW;            // per stage
  static_assert(LPW * RPL * NW == BN, "tile must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char lds[NST * SB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;

  const int group = p.Hq / p.Hkv;
  const int n_hg = p.Hq / WH;
  const int T = (p.S + ROWS - 1) / ROWS;
  const int n_pairs = (T + 1) / 2;
  const int item = xcd_remap(blockIdx.x, p.B * n_hg * n_pairs);
  const int pr = item % n_pairs;
  const int hg = (item / n_pairs) % n_hg;
  const int b = item / (n_pairs * n_hg);
  const int head = hg * WH + wave % WH;
  const int kvh = (hg * WH) / group;
  const int qblk = wave / WH;
  const float c = p.scale_log2;
  const int Sp = padded_rows(p.S);

  // Buffer descriptors over this head's K and V rows (the host checks that a
  // head's rows span less than 2^31 bytes).
  const uint32_t kss2 = (uint32_t)p.k_ss * 2u, vss2 = (uint32_t)p.v_ss * 2u;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const __bf16 *)p.k + b * p.k_sb + kvh * p.k_sh), 0,
      (int)((uint32_t)(p.S - 1) * kss2 + 2 * D), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((const __bf16 *)p.v + b * p.v_sb + kvh * p.v_sh), 0,
      (int)((uint32_t)(p.S - 1) * vss2 + 2 * D), 0x00020000);
  int lrow[LPW], lch[LPW];
#pragma unroll
  for (int q = 0; q < LPW; ++q) {
    lrow[q] = (wave * LPW + q) * RPL + lane / CPR;
    lch[q] = (lane % CPR) ^ swz<D>(lrow[q]);
  }
  const FragOffsets<D> fo(lane);

  for (int pass = 0; pass < 2; ++pass) {
    const int t = pass == 0 ? pr : T - 1 - pr;
    if (pass == 1 && t == pr) break;
    const int row0 = t * ROWS + qblk * 32;
    const int my_row = row0 + l32;
    const bool row_ok = my_row < p.S;
    const int rr = min(my_row, p.S - 1);
    const bool wave_rows = row0 < p.S;
    const int w_qmax = min(row0 + 31, p.S - 1);
    const int wg_qmax = min(t * ROWS + ROWS, p.S) - 1;

    bf16x8 qf[KS], dof[KS];
    float dsum = 0.f;   // this lane's half of D_i = sum_d dO_id O_id
    {
      const __bf16 *qr = (const __bf16 *)p.q + b * p.q_sb + head * p.q_sh + (int64_t)rr * p.q_ss + 8 * h2;
      const __bf16 *gr = (const __bf16 *)p.dout + b * p.do_sb + head * p.do_sh + (int64_t)rr * p.do_ss + 8 * h2;
      const __bf16 *orr = (const __bf16 *)p.o + b * p.o_sb + head * p.o_sh + (int64_t)rr * p.o_ss + 8 * h2;
      // Q times scale * log2(e), rounded to bf16 (as the forward forms its scores)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 raw = row_ok ? *(const bf16x8 *)(qr + 16 * ks) : bf16x8{};
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)((float)raw[e] * c);
        dof[ks] = row_ok ? *(const bf16x8 *)(gr + 16 * ks) : bf16x8{};
        const bf16x8 ov = row_ok ? *(const bf16x8 *)(orr + 16 * ks) : bf16x8{};
#pragma unroll
        for (int e = 0; e < 8; ++e) dsum = fmaf((float)ov[e], (float)dof[ks][e], dsum);
      }
    }
    // -LSE*log2(e) and -D_i of this lane's row (-inf and 0 past the last row or
    // where no key is visible: probability 0); the dK/dV kernel, launched after
    // this one, reads them from the workspace
    float nl2 = -INFINITY;
    if (row_ok) {
      const float lse = p.lse[b * p.l_sb + head * p.l_sh + (int64_t)rr * p.l_ss];
      if (lse != -INFINITY) nl2 = -lse * kLog2e;
    }
    const float nd = row_ok ? -(dsum + __shfl_xor(dsum, 32)) : 0.f;
    if (h2 == 0 && my_row < Sp) {
      float *rv = p.rowv + ((int64_t)b * p.Hq + head) * Sp * 2;
      rv[rv_index(my_row)] = nl2;
      rv[rv_index(my_row) + 16] = nd;
    }
    // the S accumulators start from -LSE * log2(e) of the lane's query (a -D
    // start for dP as well would cost 16 more registers than the kernel has)
    f32x16 sinit;
#pragma unroll
    for (int r = 0; r < 16; ++r) sinit[r] = nl2;
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

    const int nkt = p.causal ? wg_qmax / BN + 1 : (p.S + BN - 1) / BN;
    auto issue = [&](int kt, int st) {
      char *sb = lds + st * SB;
#pragma unroll
      for (int q = 0; q < LPW; ++q) {
        const uint32_t key = (uint32_t)min(kt * BN + lrow[q], p.S - 1);
        char *dst = sb + (wave * LPW + q) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void *)dst, 16, key * kss2 + 16 * lch[q], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void *)(dst + TB), 16, key * vss2 + 16 * lch[q], 0, 0, 0);
      }
    };
    auto compute = [&](int kt, int st) {
      const int k0 = kt * BN;
      if (__builtin_expect(!wave_rows || (p.causal && k0 > w_qmax), 0)) return;
      const char *sb = lds + st * SB;
      const bool full = k0 + BN <= p.S && (!p.causal || k0 + BN - 1 <= row0);
      const int lim = p.causal ? min(p.S - 1, my_row) : p.S - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (__builtin_expect(p.causal && k0 + 32 * kb > w_qmax, 0)) continue;
        const char *kt_ = sb + kb * 32 * RB;
        f32x16 s, dp = f32x16{};
        run_b128<KS>([&](int i) { return kt_ + fo.aoff[i]; },
                     [&](int i, bf16x8 a) { s = mfma32(a, qf[i], i == 0 ? sinit : s); });
        run_b128<KS>([&](int i) { return kt_ + TB + fo.aoff[i]; },
                     [&](int i, bf16x8 a) { dp = mfma32(a, dof[i], dp); });
        // lane (h2, l32) holds key k0 + 32kb + 8(r/4) + 4h2 + r%4 of query my_row;
        // keys past the limit get score -inf, so probability 0 (a uniform
        // branch: full tiles skip the compares)
        if (__builtin_expect(!full, 0)) {
          const int rel = lim - (k0 + 32 * kb + 4 * h2);
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = 8 * (r >> 2) + (r & 3) <= rel ? s[r] : -INFINITY;
        }
        bf16x8 dsk[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = __builtin_amdgcn_exp2f(s[r]);
          dsk[r >> 3][r & 7] = (__bf16)(x * (dp[r] + nd));
        }
        // dQ^T += K^T . dS^T over this block's 32 keys
        run_tr<2 * DB>([&](int i) { return kt_ + (i & 1) * 16 * RB + fo.tlo[i >> 1]; },
                       [&](int i) { return kt_ + (i & 1) * 16 * RB + fo.thi[i >> 1]; },
                       [&](int i, bf16x8 a) { acc[i >> 1] = mfma32(a, dsk[i & 1], acc[i >> 1]); });
      }
    };

    // Ring of NST stages (tile j in stage j % NST), fetched three tiles ahead;
    // past the last tile the free stage is refilled with the current tile so
    // every step has the same number of loads in flight.  Stage j+3 is the
    // stage of tile j-1, whose reads finished before the previous barrier.
    issue(0, 0);
    issue(min(1, nkt - 1), 1);
    issue(min(2, nkt - 1), 2);
    wait_vmcnt<2 * LT>();
    __builtin_amdgcn_s_barrier();
    for (int kt = 0; kt < nkt; ++kt) {
      issue(kt + 3 < nkt ? kt + 3 : kt, (kt + 3) % NST);
      compute(kt, kt % NST);
      wait_vmcnt<2 * LT>();   // this wave's part of tile kt+1 has landed
      __builtin_amdgcn_s_barrier();
    }
    wait_vmcnt<0>();   // no load into LDS may outlive the pass
    __builtin_amdgcn_s_barrier();

    if (row_ok) {
      float *dqr = p.dq + b * p.dq_sb + head * p.dq_sh + (int64_t)my_row * p.dq_ss;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = p.scale * acc[db][4 * g + e];
          *(f32x4 *)(dqr + db * 32 + 8 * g + 4 * h2) = w;
        }
    }
  }
}

// ---- dK, dV ------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void dkdv_body(const AttnBwdParams &p) {
  constexpr int NW = 4, KB = 32 * NW, QT = 64;
  constexpr int KS = D / 16, DB = D / 32, RB = 2 * D, CPR = D / 8, RPL = 64 / CPR;
  constexpr int TB = QT * RB;            // bytes of one staged Q or dO tile
  constexpr int SB = 2 * TB + 512;       // a stage: Q, dO, then the tile's row values
  constexpr int NST = 4;
  constexpr int LPW = QT / RPL / NW;     // 1 KB loads per wave and operand
  constexpr int LT = 2 * LPW + 1;        // per stage (one row-value load per wave)
  static_assert(LPW * RPL * NW == QT, "tile must split evenly over the waves");
  static_assert(QT == kRowPad, "a query tile's row values are one padded block");
  __shared__ __attribute__((aligned(1024))) char lds[NST * SB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;

  const int group = p.Hq / p.Hkv;
  const int NB = (p.S + KB - 1) / KB;
  const int n_pairs = (NB + 1) / 2;
  const int item = xcd_remap(blockIdx.x, p.B * p.Hkv * n_pairs);
  const int pr = item % n_pairs;
  const int kvh = (item / n_pairs) % p.Hkv;
  const int b = item / (n_pairs * p.Hkv);
  const float c = p.scale_log2;
  const int Sp = padded_rows(p.S);
  const int nqt = Sp / QT;
  const uint32_t qss2 = (uint32_t)p.q_ss * 2u, dss2 = (uint32_t)p.do_ss * 2u;
  const int qbytes = (int)((uint32_t)(p.S - 1) * qss2 + 2 * D);
  const int dbytes = (int)((uint32_t)(p.S - 1) * dss2 + 2 * D);
  int lrow[LPW], lch[LPW];
#pragma unroll
  for (int q = 0; q < LPW; ++q) {
    lrow[q] = (wave * LPW + q) * RPL + lane / CPR;
    lch[q] = (lane % CPR) ^ swz<D>(lrow[q]);
  }
  const FragOffsets<D> fo(lane);

  for (int pass = 0; pass < 2; ++pass) {
    const int blk = pass == 0 ? pr : NB - 1 - pr;
    if (pass == 1 && blk == pr) break;
    const int kb0 = blk * KB;
    const int kw0 = kb0 + 32 * wave;
    const int my_key = kw0 + l32;
    const bool key_ok = my_key < p.S;
    const int kk = min(my_key, p.S - 1);
    const bool wave_keys = kw0 < p.S;

    bf16x8 kf[KS], vf[KS];
    {
      const __bf16 *kr = (const __bf16 *)p.k + b * p.k_sb + kvh * p.k_sh + (int64_t)kk * p.k_ss + 8 * h2;
      const __bf16 *vr = (const __bf16 *)p.v + b * p.v_sb + kvh * p.v_sh + (int64_t)kk * p.v_ss + 8 * h2;
      // K times scale * log2(e), rounded to bf16: the scores come out in base 2
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 raw = key_ok ? *(const bf16x8 *)(kr + 16 * ks) : bf16x8{};
#pragma unroll
        for (int e = 0; e < 8; ++e) kf[ks][e] = (__bf16)((float)raw[e] * c);
        vf[ks] = key_ok ? *(const bf16x8 *)(vr + 16 * ks) : bf16x8{};
      }
    }
    f32x16 dva[DB], dka[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dva[db] = f32x16{}, dka[db] = f32x16{};

    // steps: (query head of the group, query tile) over the tiles that can see
    // a key of the block
    const int t0 = p.causal ? kb0 / QT : 0;
    const int per_head = nqt - t0;
    const int steps = group * per_head;
    auto issue = [&](int st_i, int st) {
      const int head = kvh * group + st_i / per_head;
      const int t = t0 + st_i % per_head;
      const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)((const __bf16 *)p.q + b * p.q_sb + head * p.q_sh), 0, qbytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)((const __bf16 *)p.dout + b * p.do_sb + head * p.do_sh), 0, dbytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(p.rowv + ((int64_t)b * p.Hq + head) * Sp * 2), 0, Sp * 8, 0x00020000);
      char *sb = lds + st * SB;
#pragma unroll
      for (int q = 0; q < LPW; ++q) {
        const uint32_t row = (uint32_t)min(t * QT + lrow[q], p.S - 1);
        char *dst = sb + (wave * LPW + q) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_void *)dst, 16, row * qss2 + 16 * lch[q], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (lds_void *)(dst + TB), 16, row * dss2 + 16 * lch[q], 0, 0, 0);
      }
      // 512 bytes of row values: 128 per wave, lanes 0..7
      if (lane < 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_void *)(sb + 2 * TB + 128 * wave), 16,
                                                 t * QT * 8 + 128 * wave + 16 * lane, 0, 0, 0);
    };
    auto compute = [&](int st_i, int st) {
      if (__builtin_expect(!wave_keys, 0)) return;
      const int q0 = (t0 + st_i % per_head) * QT;
      if (__builtin_expect(p.causal && q0 + QT - 1 < kw0, 0)) return;   // every query precedes every key
      const char *sb = lds + st * SB;
      const float *rv = (const float *)(sb + 2 * TB);
      // query q0 + 32qb + 8g + 4h2 + e sees key my_key iff 32qb + 8g + e >= qoff
      const int qoff = p.causal ? my_key - q0 - 4 * h2 : -(1 << 30);
      f32x16 s[2], dp[2], sinit[2], dpinit[2];
      bf16x8 pk[2][2], dsk[2][2];
      // Accumulator element r of block qb belongs to query 8(r/4) + 4h2 + r%4 of
      // the block: S starts from that query's -LSE * log2(e), or -inf where the
      // key is not visible (a uniform branch: only steps that cross the
      // diagonal compare), dP from its -D
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ri = rv_index(32 * qb + 8 * g + 4 * h2);
          const f32x4 l4 = *(const f32x4 *)(rv + ri);
          const f32x4 d4 = *(const f32x4 *)(rv + ri + 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) sinit[qb][4 * g + e] = l4[e], dpinit[qb][4 * g + e] = d4[e];
        }
      if (__builtin_expect(p.causal && q0 < kw0 + 31, 0)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sinit[qb][r] = 32 * qb + 8 * (r >> 2) + (r & 3) >= qoff ? sinit[qb][r] : -INFINITY;
      }
      // P and dS of element r (query 8(r/4) + 4h2 + r%4 of the block) of block qb
      auto elem = [&](int qb, int r) {
        const float x = __builtin_amdgcn_exp2f(s[qb][r]);
        pk[qb][r >> 3][r & 7] = (__bf16)x;
        dsk[qb][r >> 3][r & 7] = (__bf16)(x * dp[qb][r]);
      };
      constexpr int NM = 2 * KS;          // MFMAs per phase (= 4 * DB)
      constexpr int EPM = 16 / NM;        // softmax elements per MFMA
      // MFMA i of S, dP of block qb: even i -> S (A: Q rows), odd i -> dP (A: dO rows)
      auto sdp = [&](int qb, auto side) {
        auto addr = [&](int i) { return sb + qb * 32 * RB + ((i & 1) ? TB : 0) + fo.aoff[i >> 1]; };
        constexpr int A = kAhead;
        bf16x8 f[A];
#pragma unroll
        for (int i = 0; i < A; ++i) f[i] = *(const bf16x8 *)addr(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          const bf16x8 fa = f[i % A];
          if (i + A < NM) f[i % A] = *(const bf16x8 *)addr(i + A);
          if (i & 1) dp[qb] = mfma32(fa, vf[i >> 1], i == 1 ? dpinit[qb] : dp[qb]);
          else s[qb] = mfma32(fa, kf[i >> 1], i == 0 ? sinit[qb] : s[qb]);
          side(i);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // MFMA i of dV, dK of block qb: column block i / 4, half (i / 2) % 2; even i ->
      // dV (A: dO^T), odd i -> dK (A: Q^T)
      auto dvdk = [&](int qb, auto side) {
        auto lo = [&](int i) { return sb + qb * 32 * RB + ((i & 1) ? 0 : TB) + ((i >> 1) & 1) * 16 * RB + fo.tlo[i >> 2]; };
        auto hi = [&](int i) { return sb + qb * 32 * RB + ((i & 1) ? 0 : TB) + ((i >> 1) & 1) * 16 * RB + fo.thi[i >> 2]; };
        constexpr int A = kAhead;
        i16x4 fl[A], fh[A];
#pragma unroll
        for (int i = 0; i < A; ++i) fl[i] = ds_read_tr(lo(i)), fh[i] = ds_read_tr(hi(i));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          const bf16x8 fa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(fl[i % A], fh[i % A], 0, 1, 2, 3, 4, 5, 6, 7));
          if (i + A < NM) fl[i % A] = ds_read_tr(lo(i + A)), fh[i % A] = ds_read_tr(hi(i + A));
          const int db = i >> 2, hh = (i >> 1) & 1;
          if (i & 1) dka[db] = mfma32(fa, dsk[qb][hh], dka[db]);
          else dva[db] = mfma32(fa, pk[qb][hh], dva[db]);
          side(i);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      auto none = [](int) {};
      sdp(0, none);
      sdp(1, [&](int i) {
#pragma unroll
        for (int k = 0; k < EPM; ++k) elem(0, i * EPM + k);
      });
      dvdk(0, [&](int i) {
#pragma unroll
        for (int k = 0; k < EPM; ++k) elem(1, i * EPM + k);
      });
      dvdk(1, none);
    };

    // Same ring as the dq kernel (steps >= 1: the last query tile sees every key).
    issue(0, 0);
    issue(min(1, steps - 1), 1);
    issue(min(2, steps - 1), 2);
    wait_vmcnt<2 * LT>();
    __builtin_amdgcn_s_barrier();
    for (int st_i = 0; st_i < steps; ++st_i) {
      issue(st_i + 3 < steps ? st_i + 3 : st_i, (st_i + 3) % NST);
      compute(st_i, st_i % NST);
      wait_vmcnt<2 * LT>();
      __builtin_amdgcn_s_barrier();
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();

    if (key_ok) {
      float *dkr = p.dk + b * p.dk_sb + kvh * p.dk_sh + (int64_t)my_key * p.dk_ss;
      float *dvr = p.dv + b * p.dv_sb + kvh * p.dv_sh + (int64_t)my_key * p.dv_ss;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 wk, wv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            wk[e] = p.scale * dka[db][4 * g + e];
            wv[e] = dva[db][4 * g + e];
          }
          *(f32x4 *)(dkr + db * 32 + 8 * g + 4 * h2) = wk;
          *(f32x4 *)(dvr + db * 32 + 8 * g + 4 * h2) = wv;
        }
    }
  }
}

// One plain kernel per configuration (the bodies are templates).
#define CHAIN_BWD_KERNELS(D)                                                                            \
  __global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2)))            \
  void attn_bwd_dq_kernel_d##D##_g1(const AttnBwdParams p) { dq_body<D, 1>(p); }                        \
  __global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2)))            \
  void attn_bwd_dq_kernel_d##D##_g2(const AttnBwdParams p) { dq_body<D, 2>(p); }                        \
  __global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2)))            \
  void attn_bwd_dq_kernel_d##D##_g4(const AttnBwdParams p) { dq_body<D, 4>(p); }                        \
  __global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))          \
  void attn_bwd_dkdv_kernel_d##D(const AttnBwdParams p) { dkdv_body<D>(p); }
CHAIN_BWD_KERNELS(64)
CHAIN_BWD_KERNELS(128)
#undef CHAIN_BWD_KERNELS

template <int D>
hipError_t launch_d(const AttnBwdParams &p, hipStream_t s) {
  const int group = p.Hq / p.Hkv;
  const int wh = group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
  const int rows_t = 32 * (8 / wh);
  const int T = (p.S + rows_t - 1) / rows_t;
  const dim3 gq(p.B * (p.Hq / wh) * ((T + 1) / 2));
  if (wh == 4) hipLaunchKernelGGL((D == 64 ? attn_bwd_dq_kernel_d64_g4 : attn_bwd_dq_kernel_d128_g4), gq, dim3(512), 0, s, p);
  else if (wh == 2) hipLaunchKernelGGL((D == 64 ? attn_bwd_dq_kernel_d64_g2 : attn_bwd_dq_kernel_d128_g2), gq, dim3(512), 0, s, p);
  else hipLaunchKernelGGL((D == 64 ? attn_bwd_dq_kernel_d64_g1 : attn_bwd_dq_kernel_d128_g1), gq, dim3(512), 0, s, p);
  const int NB = (p.S + 127) / 128;
  const dim3 gk(p.B * p.Hkv * ((NB + 1) / 2));
  hipLaunchKernelGGL((D == 64 ? attn_bwd_dkdv_kernel_d64 : attn_bwd_dkdv_kernel_d128), gk, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const AttnBwdParams &p, int D, hipStream_t s) {
  if (p.B == 0 || p.Hq == 0 || p.S == 0) return hipSuccess;
  return D == 64 ? launch_d<64>(p, s) : launch_d<128>(p, s);
}

}  // namespace chain
