// Causal / GQA attention forward on bf16 MFMA tiles (gfx950).
//
// Computes the chain O = f(Q.K^T).V of the METP article (abstract) with f the
// scaled, masked row softmax, over key/value ranges visited chunk by chunk (the
// zigzag chunks of the TSP article, "Lo que realmente significa plegar"; the
// context chunks of the 2D-Attention summary, "Introduciendo la Atencion 2D"),
// merging chunks with an online softmax that carries a reference max m and the
// sum l in registers.  GQA (2D-Attention summary, "Comprendiendo la
// Arquitectura de los LLMs"): the waves of one workgroup take query heads of
// the same key/value head, so a staged key/value tile serves all of them.
//
// Per wave: 32 query rows of one head.  S^T = K.Q^T with v_mfma_f32_32x32x16_bf16
// (keys are the M index, queries the N index), so each lane owns one query
// column and 16 key rows per 32-key block: the row max is an in-lane reduction
// plus one exchange between lane halves (v_permlane32_swap), the row sum stays
// per lane until the epilogue.  The S^T accumulator, rounded to bf16, is
// directly the B operand of O^T += V^T.P^T: within each 16-key step lane half h
// holds keys {4h..4h+3, 8+4h..8+4h+3}, and the V^T operand is read in that
// order from the row-major V tile with ds_read_b64_tr_b16.
//
// Eight waves per workgroup (two per SIMD) share each staged 64-key K/V tile.
// Tiles reach LDS by buffer loads that write LDS directly (64 lanes x 16 bytes
// per wave-level load, no staging registers, no LDS write instructions) into a
// ring of four stages fetched three tiles ahead; one barrier per tile.  Staged
// rows are not padded: 16-byte chunks are XOR-swizzled per row so that the
// 16-byte K fragment reads and the transposing V reads each hit distinct bank
// groups.  Inside each MFMA run the LDS fragments are read kAhead MFMAs ahead
// of use (pinned with scheduling barriers) and the wave raises its issue
// priority, so the other wave on the SIMD fills the VALU (softmax) while this
// one feeds the matrix core.  The reference max is raised only when a row's max grows past it by
// more than 2^8 (exact: O and l share the reference), so the O rescale is rare.
// The row sum l adds the unrounded f32 probabilities, so the LSE stays exact to
// f32 rounding whatever chunk order the tiles are visited in.
#include "internal.h"

namespace chain {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 64;          // keys per tile
constexpr float kTau = 8.0f;    // lazy rescale threshold (base-2 exponent)
constexpr float kLaneSumMax = 256.0f;   // 2^kTau
constexpr int kAhead = 4;       // LDS fragments in flight ahead of their MFMA

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: in each group of 16 lanes, lane i receives element i%4
// of the 4-element rows addressed by lanes 4e + i/4, e = 0..3.  The restrict
// qualifier gives the read alias-scope information once inlined; without it the
// compiler cannot tell the read from the direct-to-LDS loads in flight and
// waits for all of them (vmcnt(0)) before every P.V run.  Every tile a read
// touches has landed and passed a barrier, so no such wait is needed.
__device__ inline i16x4 ds_read_tr(const __bf16 *__restrict__ p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

// Max over the two lane halves (lanes l and l^32 hold the same query).
__device__ inline float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

template <int D, int NW, int WH>
__device__ __forceinline__ void attn_mfma_bf16(const AttnParams &p) {
  constexpr int WQ = NW / WH;               // 32-row query blocks per head
  constexpr int ROWS = 32 * WQ;             // query positions per tile
  constexpr int KS = D / 16;                // k-steps of K.Q^T
  constexpr int DB = D / 32;                // 32-wide blocks of O^T
  constexpr int RB = 2 * D;                 // bytes per key row of a staged tile
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int RPL = 64 / CPR;             // rows per 1 KB wave load
  constexpr int TB = BN * RB;               // bytes of one staged K or V tile
  constexpr int SB = 2 * TB;                // a stage: the K tile, then the V tile
  constexpr int NST = 4;                    // stages in the ring
  constexpr int LPW = BN / RPL / NW;        // 1 KB loads per wave, operand and tile
  constexpr int LT = 2 * LPW;               // per tile
  static_assert(LPW * RPL * NW == BN, "tile must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char lds[NST * SB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;

  // ---- work item: (batch, head group, pair of query tiles t and T-1-t)
  const int group = p.Hq / p.Hkv;
  const int n_hg = p.Hq / WH;
  const int T = (p.Sq + ROWS - 1) / ROWS;
  const int n_pairs = (T + 1) / 2;
  const int n_items = p.B * n_hg * n_pairs;
  const int item = xcd_remap(blockIdx.x, n_items);
  const int pr = item % n_pairs;
  const int hg = (item / n_pairs) % n_hg;
  const int b = item / (n_pairs * n_hg);
  const int head = hg * WH + wave % WH;
  const int kvh = (hg * WH) / group;
  const int qblk = wave / WH;

  const __bf16 *kbase = (const __bf16 *)p.k + b * p.k_sb + kvh * p.k_sh;
  const __bf16 *vbase = (const __bf16 *)p.v + b * p.v_sb + kvh * p.v_sh;
  const float c = p.scale_log2;
  // Buffer descriptors over this head's K and V rows (byte offsets fit 32 bits:
  // the host checks that a head's rows span less than 2^31 bytes).
  const uint32_t kss2 = (uint32_t)p.k_ss * 2u, vss2 = (uint32_t)p.v_ss * 2u;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)kbase, 0, (int)((uint32_t)(p.Sk - 1) * kss2 + 2 * D), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)vbase, 0, (int)((uint32_t)(p.Sk - 1) * vss2 + 2 * D), 0x00020000);

  // Rows of a staged tile are not padded: 16-byte chunk c of key row r sits at
  // chunk c ^ kswz(r) in K and c ^ vswz(r) in V.  kswz spreads the 16-byte
  // fragment reads of 16 consecutive keys over 16 distinct bank groups; vswz
  // does the same for the 4 rows x 4 chunks a transposing read touches per
  // 32 lanes.  The load side picks which global chunk each lane fetches, so the
  // swizzle costs nothing there.
  auto kswz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto vswz = [](int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
  int lrow[LPW], kch[LPW], vch[LPW];
#pragma unroll
  for (int q = 0; q < LPW; ++q) {
    lrow[q] = (wave * LPW + q) * RPL + lane / CPR;
    kch[q] = (lane % CPR) ^ kswz(lrow[q]);
    vch[q] = (lane % CPR) ^ vswz(lrow[q]);
  }
  // Per-lane byte offsets of the MFMA fragments within a stage.
  int koff[KS], voff[DB];
  {
    const int xk = kswz(l32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = l32 * RB + (((2 * ks + h2) ^ xk) << 4);
    const int trow = 4 * h2 + ((lane & 15) >> 2);
    const int ylane = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int xv = D == 128 ? (trow & 3) : ((trow >> 1) & 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) voff[db] = TB + trow * RB + ((4 * (db ^ xv) + ylane) << 4) + 8 * (lane & 1);
  }

  for (int pass = 0; pass < 2; ++pass) {
    const int t = pass == 0 ? pr : T - 1 - pr;
    if (pass == 1 && t == pr) break;
    const int wg_row0 = t * ROWS;
    const int wg_last = min(wg_row0 + ROWS, p.Sq) - 1;
    const int32_t wg_qmax = row_position(p.qruns, wg_last);
    const int row0 = wg_row0 + qblk * 32;
    const bool wave_rows = row0 < p.Sq;
    const int w_last = min(row0 + 31, p.Sq - 1);
    const int32_t w_qmin = row_position(p.qruns, min(row0, p.Sq - 1));
    const int32_t w_qmax = row_position(p.qruns, w_last);
    const int my_row = row0 + l32;
    const bool row_ok = my_row < p.Sq;
    const int32_t my_qpos = row_position(p.qruns, min(my_row, p.Sq - 1));

    bf16x8 qf[KS];
    {
      const __bf16 *qrow = (const __bf16 *)p.q + b * p.q_sb + head * p.q_sh +
                           (int64_t)min(my_row, p.Sq - 1) * p.q_ss + 8 * h2;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = *(const bf16x8 *)(qrow + ks * 16);
        if (!row_ok) qf[ks] = bf16x8{};
      }
    }
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    float m = -INFINITY, l = 0.f;

    // ---- tile iterator (uniform over the workgroup)
    auto range_live = [&](int ri) {
      return p.kr.end[ri] > p.kr.beg[ri] && (!p.causal || p.kr.beg[ri] + p.kr.pos_off[ri] <= wg_qmax);
    };
    auto advance = [&](int &ri, int &k0) -> bool {
      k0 += BN;
      if (k0 < p.kr.end[ri] && (!p.causal || k0 + p.kr.pos_off[ri] <= wg_qmax)) return true;
      for (++ri; ri < p.kr.n; ++ri)
        if (range_live(ri)) { k0 = p.kr.beg[ri]; return true; }
      return false;
    };
    struct Tl { int ri, k0, kend, off; bool valid; };   // range end and position offset cached
    auto first_tile = [&]() -> Tl {
      for (int r = 0; r < p.kr.n; ++r)
        if (range_live(r)) return Tl{r, p.kr.beg[r], p.kr.end[r], p.kr.pos_off[r], true};
      return Tl{0, 0, 0, 0, false};
    };
    auto next_tile = [&](Tl x) -> Tl {
      if (!x.valid) return x;
      int r = x.ri, k = x.k0;
      return advance(r, k) ? Tl{r, k, p.kr.end[r], p.kr.pos_off[r], true} : Tl{0, 0, 0, 0, false};
    };
    // Direct-to-LDS loads of one tile into stage st: each wave-level load puts
    // 64 lanes x 16 bytes (RPL key rows) into LDS.  Keys past the range end
    // read its last key; zero_tail clears them once they have landed.
    auto issue = [&](const Tl &x, int st) {
      char *sb = lds + st * SB;
      const int kend = x.kend;
#pragma unroll
      for (int q = 0; q < LPW; ++q) {
        const uint32_t key = (uint32_t)min(x.k0 + lrow[q], kend - 1);
        char *dst = sb + (wave * LPW + q) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void *)dst, 16,
                                                 key * kss2 + 16 * kch[q], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void *)(dst + TB), 16,
                                                 key * vss2 + 16 * vch[q], 0, 0, 0);
      }
    };
    auto zero_tail = [&](const Tl &x, int st) {
      const int kend = x.kend;
      char *sb = lds + st * SB + lane * 16;
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int q = 0; q < LPW; ++q)
        if (x.k0 + lrow[q] >= kend) {
          *(u32x4 *)(sb + (wave * LPW + q) * 1024) = z;
          *(u32x4 *)(sb + TB + (wave * LPW + q) * 1024) = z;
        }
    };
    auto compute = [&](const Tl &x, const int st) {
      const int k0 = x.k0;
      // ---- compute on the staged tile
      const int off = x.off;
      const int nvalid = min(BN, x.kend - k0);
      const int cls = classify_tile(p.causal, w_qmin, w_qmax, k0 + off, k0 + nvalid - 1 + off, nvalid < BN);
      if (wave_rows && cls != TILE_SKIP) {
        const char *sb = lds + st * SB;
        f32x16 s[2] = {f32x16{}, f32x16{}};
        __builtin_amdgcn_s_setprio(1);
        {
          constexpr int N = 2 * KS;
          auto addr = [&](int i) { return sb + koff[i >> 1] + (i & 1) * 32 * RB; };
          bf16x8 kf[kAhead];
#pragma unroll
          for (int i = 0; i < kAhead; ++i) kf[i] = *(const bf16x8 *)addr(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < N; ++i) {
            const bf16x8 a = kf[i % kAhead];
            if (i + kAhead < N) kf[i % kAhead] = *(const bf16x8 *)addr(i + kAhead);
            s[i & 1] = mfma32(a, qf[i >> 1], s[i & 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        if (cls == TILE_DIAG) {
          // key of register r in lane half h2 is kb*32 + 8*(r/4) + 4*h2 + r%4: compare
          // its compile-time part with per-lane limits (branch-free selects)
          const int lim_c = p.causal ? my_qpos - k0 - off - 4 * h2 : BN;
          const int lim = min(nvalid - 1 - 4 * h2, lim_c);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kr = kb * 32 + 8 * (r >> 2) + (r & 3);
              s[kb][r] = kr <= lim ? s[kb][r] : -INFINITY;
            }
        }
        // Fast path: probabilities against the current reference.  The row max
        // only decides whether the reference must rise (a term above 2^kTau); a
        // lane sum of at most 2^kTau proves no term is, so the max is computed
        // (and the rule below applied) only when some lane sum exceeds it, or
        // before the first reference exists.
        float rs = 0.f;
        bf16x8 pk[2][2];
        bool slow = __any(m == -INFINITY);
        if (!slow) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -m));
              rs += e;
              pk[kb][r >> 3][r & 7] = (__bf16)e;
            }
          slow = __any(!(rs <= kLaneSumMax));
        }
        if (slow) {
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
          // the reference max is raised only when the row max exceeds it by more
          // than 2^kTau (exact: O and l share the reference); the O rescale is rare
          const float tmax = pair_max(mx) * c;
          if (__any(tmax > m + kTau)) {
            const float m_new = fmaxf(m, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m - (m_new == -INFINITY ? 0.f : m_new));
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] *= alpha;
          }
          const float m_use = m == -INFINITY ? 0.f : m;
          rs = 0.f;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -m_use));
              rs += e;
              pk[kb][r >> 3][r & 7] = (__bf16)e;
            }
        }
        l += rs;
        // O^T += V^T . P^T
        __builtin_amdgcn_s_setprio(1);
        {
          constexpr int N = 4 * DB;
          auto addr = [&](int i) {
            const int db = i >> 2, kb = (i >> 1) & 1, hh = i & 1;
            return (const __bf16 *)(sb + voff[db] + (kb * 32 + 16 * hh) * RB);
          };
          i16x4 vlo[kAhead], vhi[kAhead];
#pragma unroll
          for (int i = 0; i < kAhead; ++i) {
            vlo[i] = ds_read_tr(addr(i));
            vhi[i] = ds_read_tr(addr(i) + 8 * D);
          }
#pragma unroll
          for (int i = 0; i < N; ++i) {
            const i16x8 a16 = __builtin_shufflevector(vlo[i % kAhead], vhi[i % kAhead], 0, 1, 2, 3, 4, 5, 6, 7);
            if (i + kAhead < N) {
              vlo[i % kAhead] = ds_read_tr(addr(i + kAhead));
              vhi[i % kAhead] = ds_read_tr(addr(i + kAhead) + 8 * D);
            }
            acc[i >> 2] = mfma32(__builtin_bit_cast(bf16x8, a16), pk[(i >> 1) & 1][i & 1], acc[i >> 2]);
        __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };

    // Ring of NST stages (tile j in stage j % NST), fetched three tiles ahead.
    // Past the last tile the free stage is refilled with the current tile, so
    // every step has the same number of loads in flight.  Stage j+3 reuses the
    // buffer of tile j-1, whose reads finished before the previous barrier.
    Tl w0 = first_tile(), w1 = next_tile(w0), w2 = next_tile(w1), w3 = next_tile(w2);
    if (w0.valid) {
      issue(w0, 0);
      issue(w1.valid ? w1 : w0, 1);
      issue(w2.valid ? w2 : w0, 2);
      wait_vmcnt<2 * LT>();
      if (w0.k0 + BN > w0.kend) zero_tail(w0, 0);
    }
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    int j = 0;
    while (w0.valid) {
      issue(w3.valid ? w3 : w0, (j + 3) % NST);
      compute(w0, j % NST);
      wait_vmcnt<2 * LT>();   // this wave's part of tile j+1 has landed
      if (w1.valid && w1.k0 + BN > w1.kend) zero_tail(w1, (j + 1) % NST);
      wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();
      w0 = w1;
      w1 = w2;
      w2 = w3;
      w3 = next_tile(w3);
      ++j;
    }
    wait_vmcnt<0>();   // no load into LDS may outlive the pass
    __builtin_amdgcn_s_barrier();

    // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l)
    const float lt = pair_sum(l);
    if (row_ok) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int64_t orow = b * p.o_sb + head * p.o_sh + (int64_t)my_row * p.o_ss;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = db * 32 + 8 * g + 4 * h2;
          const float o0 = acc[db][4 * g] * inv, o1 = acc[db][4 * g + 1] * inv;
          const float o2 = acc[db][4 * g + 2] * inv, o3 = acc[db][4 * g + 3] * inv;
          if (p.o_f32) {
            *(float4 *)((float *)p.o + orow + d0) = make_float4(o0, o1, o2, o3);
          } else {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 w = {(__bf16)o0, (__bf16)o1, (__bf16)o2, (__bf16)o3};
            *(bf16x4 *)((__bf16 *)p.o + orow + d0) = w;
          }
        }
      if (h2 == 0)
        p.lse[b * p.l_sb + head * p.l_sh + (int64_t)my_row * p.l_ss] =
            lt > 0.f ? (m + log2f(lt)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

// One plain kernel per configuration (the body is a template).
#define CHAIN_ATTN_KERNEL(D, WH)                                                               \
  __global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2))) \
  void attn_mfma_bf16_kernel_d##D##_g##WH(const AttnParams p) { attn_mfma_bf16<D, 8, WH>(p); }
CHAIN_ATTN_KERNEL(64, 1)
CHAIN_ATTN_KERNEL(64, 2)
CHAIN_ATTN_KERNEL(64, 4)
CHAIN_ATTN_KERNEL(128, 1)
CHAIN_ATTN_KERNEL(128, 2)
CHAIN_ATTN_KERNEL(128, 4)
#undef CHAIN_ATTN_KERNEL

// Workgroups: pairs of 64-row query tiles of WH query heads (8 waves of 32 rows).
template <int D>
hipError_t launch_d(const AttnParams &p, hipStream_t s) {
  const int group = p.Hq / p.Hkv;
  const int wh = group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
  const int rows = 32 * (8 / wh);
  const int T = (p.Sq + rows - 1) / rows;
  const int items = p.B * (p.Hq / wh) * ((T + 1) / 2);
  const dim3 grid(items), block(512);
  if (D == 64) {
    if (wh == 4) hipLaunchKernelGGL(attn_mfma_bf16_kernel_d64_g4, grid, block, 0, s, p);
    else if (wh == 2) hipLaunchKernelGGL(attn_mfma_bf16_kernel_d64_g2, grid, block, 0, s, p);
    else hipLaunchKernelGGL(attn_mfma_bf16_kernel_d64_g1, grid, block, 0, s, p);
  } else {
    if (wh == 4) hipLaunchKernelGGL(attn_mfma_bf16_kernel_d128_g4, grid, block, 0, s, p);
    else if (wh == 2) hipLaunchKernelGGL(attn_mfma_bf16_kernel_d128_g2, grid, block, 0, s, p);
    else hipLaunchKernelGGL(attn_mfma_bf16_kernel_d128_g1, grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma_bf16(const AttnParams &p, int D, hipStream_t s) {
  return D == 64 ? launch_d<64>(p, s) : launch_d<128>(p, s);
}

}  // namespace chain
