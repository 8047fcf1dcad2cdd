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
// Eight waves per workgroup (two per SIMD: waves w and w+4) share each staged
// 64-key K/V tile.  They run a ping-pong schedule: every wave alternates an
// MFMA phase (K.Q^T of tile j, then P.V of tile j-1) and a softmax phase (tile
// j), waves 4-7 one phase behind waves 0-3, with a workgroup barrier between
// phases, so on each SIMD one wave's MFMA run meets the other wave's softmax.
// Tiles reach LDS by buffer loads that write LDS directly (64 lanes x 16 bytes
// per wave-level load, no staging registers, no LDS write instructions) into a
// K ring and a V ring of four stages each: at the start of softmax phase j,
// waves 0-3 issue all of tile j+3's K and waves 4-7 all of tile j+3's V.
// Staged rows are not padded: 16-byte chunks are XOR-swizzled per row so that
// the 16-byte K fragment reads and the transposing V reads each hit distinct
// bank groups.  Inside each MFMA run the LDS fragments are read kAhead MFMAs
// ahead of use (pinned with scheduling barriers); the first ones of both runs
// of a phase are read at the end of the softmax phase before it.  Scalar
// branches cost tens of cycles even when not taken (about twice that when
// taken), so the tile loop keeps them few and marks the rare paths (masked
// tiles, the slow softmax path, range switches, V tails) unlikely, so that the
// common path falls through every branch.
//
// Q is multiplied by scale * log2(e) and rounded to bf16 once per query tile,
// and each K.Q^T accumulator starts from minus the row's reference max m, so
// the MFMA delivers the base-2 score minus the reference and a probability is
// one exp2: the softmax costs 32 exp2, 32 adds and 16 packs per 64-key tile and
// wave.  The reference is raised only when a row's max grows past it by more
// than 2^8 (exact: O and l share the reference), so the O rescale is rare.  The
// row sum l adds the unrounded f32 probabilities.
#include <type_traits>

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
  static_assert(NW == 8, "two groups of four waves: one wave of each group per SIMD");
  constexpr int WQ = NW / WH;               // 32-row query blocks per head
  constexpr int ROWS = 32 * WQ;             // query positions per tile
  constexpr int KS = D / 16;                // k-steps of K.Q^T
  constexpr int DB = D / 32;                // 32-wide blocks of O^T
  constexpr int RB = 2 * D;                 // bytes per key row of a staged tile
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int RPL = 64 / CPR;             // rows per 1 KB wave load
  constexpr int TB = BN * RB;               // bytes of one staged K or V tile
  constexpr int NST = 4;                    // stages in each of the K and V rings
  constexpr int LPW = BN / RPL / NW;        // 1 KB loads per wave, operand and tile
  static_assert(LPW * RPL * NW == BN, "tile must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char lds[2 * NST * TB];
  char *const kring = lds;
  char *const vring = lds + NST * TB;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  // Waves w and w+4 share a SIMD; group 0 is waves 0-3, group 1 waves 4-7.
  const int grp = wave >> 2;

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
  // Byte offsets of key rows from these bases fit 32 bits: the host checks
  // that a head's rows span less than 2^31 bytes.
  const uint32_t kss2 = (uint32_t)p.k_ss * 2u, vss2 = (uint32_t)p.v_ss * 2u;
  const char *kb8 = (const char *)kbase, *vb8 = (const char *)vbase;

  // Rows of a staged tile are not padded: 16-byte chunk c of key row r sits at
  // chunk c ^ kswz(r) in K and c ^ vswz(r) in V.  kswz spreads the 16-byte
  // fragment reads of 16 consecutive keys over 16 distinct bank groups; vswz
  // does the same for the 4 rows x 4 chunks a transposing read touches per
  // 32 lanes.  The load side picks which global chunk each lane fetches, so the
  // swizzle costs nothing there.
  auto kswz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto vswz = [](int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
  // Each group of four waves loads one operand of every tile: group 0 all of
  // K, group 1 all of V (LO loads of 1 KB per wave and tile).  lo: per-lane byte
  // offsets of a whole tile's loads from its first key.
  constexpr int LO = 2 * LPW;
  const int w4 = wave & 3;
  const char *const own_b8 = grp == 0 ? kb8 : vb8;
  const uint32_t own_ss2 = grp == 0 ? kss2 : vss2;
  int lrow[LO], ldo[LO];
#pragma unroll
  for (int q = 0; q < LO; ++q) {
    lrow[q] = (w4 * LO + q) * RPL + lane / CPR;
    const int ch = (lane % CPR) ^ (grp == 0 ? kswz(lrow[q]) : vswz(lrow[q]));
    ldo[q] = lrow[q] * own_ss2 + 16 * ch;
  }
  // Per-lane byte offsets of the MFMA fragments within a K or a V stage.
  int koff[KS], voff[DB];
  {
    const int xk = kswz(l32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = l32 * RB + (((2 * ks + h2) ^ xk) << 4);
    const int trow = 4 * h2 + ((lane & 15) >> 2);
    const int ylane = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int xv = D == 128 ? (trow & 3) : ((trow >> 1) & 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) voff[db] = trow * RB + ((4 * (db ^ xv) + ylane) << 4) + 8 * (lane & 1);
    // Hide the offsets' known bits: otherwise the compiler may turn offset +
    // stage constant into an OR per read instead of one add and immediate offsets.
#pragma unroll
    for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(voff[db]));
  }

  // ---- the two passes of an item (query tiles pr and T-1-pr) share one body
  // and the state below, which set_pass fills for query tile t.  Pass 1's Q
  // rows and first tiles are fetched before pass 0's outputs are stored, so
  // they do not queue behind the stores.
  int wg_qmax = 0, row0 = 0, my_row = 0, n = 0;
  int32_t w_qmin = 0, w_qmax = 0, my_qpos = 0;
  bool wave_rows = false, row_ok = false;
  bf16x8 qraw[KS], qf[KS];

  // ---- tile iterators (wave-uniform).  Tiles of BN keys are cut inside each
  // key range, up to the last key position this tile's queries can see (stop);
  // n counts them.  Each wave steps two iterators: cur (the tile it computes)
  // and ld (the tile whose K, group 0, or V, group 1, it loads next).  All that
  // a step needs is precomputed when an iterator enters a range (rare), so a
  // step within a range is a few scalar adds and compares behind one branch:
  //   kskip, kdiag: a tile from k0 >= kskip on is skipped by this wave, from
  //     k0 >= kdiag on masked (the causal diagonal or the range's ragged end);
  //   kzt: from k0 >= kzt on, group 1 clears V rows past the range end;
  //   base, rem: the buffer descriptor of the tile's own-operand rows (its
  //     first row, and the bytes up to the range end), advanced by dstep;
  //   left: tiles of the range after this one (the range switch when < 0).
  // Past the last tile ld repeats the first tile (dstep 0) and cur is skipped.
  struct It {
    int ri, k0, left, kend, off;   // ri == p.kr.n: past the last tile
    int kskip, kdiag, kzt;
    const char *base;
    int rem, dstep;
  };
  It first{}, cur{}, ld{};
  auto range_stop = [&](int r) {
    return p.causal ? min(p.kr.end[r], wg_qmax - p.kr.pos_off[r] + 1) : p.kr.end[r];
  };
  auto seek = [&](int r) -> It {   // first tile of the first live range at or after r
    for (; r < p.kr.n; ++r) {
      const int st = range_stop(r);
      const int k0 = p.kr.beg[r], kend = p.kr.end[r], off = p.kr.pos_off[r];
      if (st > k0) {
        // classify_tile's tests as thresholds on k0: skipped once the first key
        // passes the wave's last query; masked once the last key passes its
        // first query, or the tile is cut short by the range end
        const int kskip = !wave_rows ? INT_MIN : p.causal ? w_qmax - off + 1 : INT_MAX;
        const int kdiag = min(kend - BN + 1, p.causal ? w_qmin - off - BN + 2 : INT_MAX);
        return It{r, k0, (st - k0 - 1) / BN, kend, off, kskip, kdiag, grp == 1 ? kend - BN + 1 : INT_MAX,
                  own_b8 + (uint32_t)k0 * own_ss2, (int)((uint32_t)(kend - k0 - 1) * own_ss2 + 2 * D),
                  (int)((uint32_t)BN * own_ss2)};
      }
    }
    return It{p.kr.n, 0, INT_MAX, 0, 0, INT_MIN, INT_MIN, INT_MAX, first.base, first.rem, 0};   // never switches
  };
  auto step_ld = [&](It &l) {
    l.left -= 1;
    l.base += (uint32_t)l.dstep;
    l.rem -= l.dstep;
  };
  auto step_one = [&](It &x) {
    step_ld(x);
    if (x.left < 0) x = seek(x.ri + 1);
  };
  auto step2 = [&](It &c, It &l) {
    c.k0 += BN;
    c.left -= 1;
    step_ld(l);
    if (__builtin_expect(min(c.left, l.left) < 0, 0)) {
      if (c.left < 0) c = seek(c.ri + 1);
      if (l.left < 0) l = seek(l.ri + 1);
    }
  };
  // What this wave does with a tile: skip it, take it whole, or mask it (the
  // tests of classify_tile, precomputed as thresholds).
  auto tile_class = [&](const It &x) -> int {
    return x.k0 >= x.kskip ? TILE_SKIP : x.k0 >= x.kdiag ? TILE_DIAG : TILE_FULL;
  };
  // Direct-to-LDS loads of one operand of one tile into a ring stage: each
  // wave-level load puts 64 lanes x 16 bytes (RPL key rows) into LDS.  The
  // buffer descriptor starts at the tile's first key row and ends at its
  // range end, so the same branch-free loads serve whole tiles and tiles cut
  // short: keys past the range end are out of the buffer and read as zero
  // (their scores are masked, their V rows cleared as well).
  auto issue = [&](const It &x, char *stage) {   // this wave's part of its group's operand
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)x.base, 0, x.rem, 0x00020000);
#pragma unroll
    for (int q = 0; q < LO; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(stage + (w4 * LO + q) * 1024),
                                               16, ldo[q], 0, 0, 0);
  };
  // V rows past a range end are cleared once this wave's own loads of them
  // have landed, so that a masked key multiplies zeros whatever the input holds.
  auto zero_v_tail = [&](const It &x, char *stage) {
    if (__builtin_expect(x.k0 >= x.kzt, 0)) {
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int q = 0; q < LO; ++q)
        if (x.k0 + lrow[q] >= x.kend) *(u32x4 *)(stage + (w4 * LO + q) * 1024 + lane * 16) = z;
      wait_lgkmcnt0();
    }
  };

  auto set_pass = [&](int t) {
    const int wg_row0 = t * ROWS;
    const int wg_last = min(wg_row0 + ROWS, p.Sq) - 1;
    wg_qmax = row_position(p.qruns, wg_last);
    row0 = wg_row0 + qblk * 32;
    wave_rows = row0 < p.Sq;
    const int w_last = min(row0 + 31, p.Sq - 1);
    w_qmin = row_position(p.qruns, min(row0, p.Sq - 1));
    w_qmax = row_position(p.qruns, w_last);
    my_row = row0 + l32;
    row_ok = my_row < p.Sq;
    my_qpos = row_position(p.qruns, min(my_row, p.Sq - 1));
    n = 0;
    for (int r = 0; r < p.kr.n; ++r) {
      const int st = range_stop(r);
      if (st > p.kr.beg[r]) n += (st - p.kr.beg[r] + BN - 1) / BN;
    }
  };
  // The pass's Q rows; convert_q then forms Q times scale * log2(e), rounded
  // to bf16, so the products come out of the MFMA in base-2 units.
  auto load_q = [&] {
    const __bf16 *qrow = (const __bf16 *)p.q + b * p.q_sb + head * p.q_sh +
                         (int64_t)min(my_row, p.Sq - 1) * p.q_ss + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = *(const bf16x8 *)(qrow + ks * 16);
  };
  auto convert_q = [&] {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = row_ok ? (__bf16)((float)qraw[ks][e] * c) : (__bf16)0.f;
  };
  // The ring's first loads of a pass: group 0 K, group 1 V of tiles 0, 1 and
  // 2.  cur: tile j (K.Q^T, softmax); ld: tile j+3, whose K or V is loaded in
  // S_j.  Past the last tile the loads repeat the first tile into the free
  // stages, so every step has the same loads in flight.
  char *const own_ring = grp == 0 ? kring : vring;
  auto start_tiles = [&] {
    if (n > 0) {
      first = seek(0);
      cur = first;
      ld = first;
      issue(ld, own_ring);
      step_one(ld);
      issue(ld, own_ring + TB);
      step_one(ld);
      issue(ld, own_ring + 2 * TB);
      step_one(ld);
    }
  };

  const bool two = T - 1 - pr != pr;   // the middle tile of an odd count is one pass
  set_pass(pr);
  load_q();
  start_tiles();
  convert_q();
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1 && !two) break;
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    // m: the reference max (base 2) of this lane's row, -inf until set; the K.Q^T
    // accumulators start from -mu, mu = m (0 while m is -inf), so they hold the
    // scores minus the reference and the fast path's probability is one exp2.
    float m = -INFINITY, l = 0.f, mu = 0.f;
    f32x16 mref = f32x16{};   // -mu in every element
    // the fast path's lane-sum bound: kLaneSumMax once every lane of the wave
    // holds a finite reference max, -1 (no lane passes) before that
    float sum_bound = -1.f;
    f32x16 s[2];
    bf16x8 pk[2][2];

    // MFMA run: NQ products of S^T = K.Q^T on a K stage, then NP products of
    // O^T += V^T.P^T on a V stage (the previous tile's P).  LDS fragments are
    // read kAhead MFMAs ahead of use.  With pre = true a run takes its first
    // kAhead fragments from fq (a K.Q^T run) or fv (a P.V run), read at the end
    // of the softmax step before it, so their LDS latency passes under the
    // barrier and (for fv) under the K.Q^T run.
    bf16x8 fq[kAhead], fv[kAhead];
    auto kfrag = [&](const char *ks, int i) -> bf16x8 {
      return *(const bf16x8 *)(ks + koff[i >> 1] + (i & 1) * 32 * RB);
    };
    auto vfrag = [&](const char *vs, int k) -> bf16x8 {
      const __bf16 *a = (const __bf16 *)(vs + voff[k >> 2] + (((k >> 1) & 1) * 32 + 16 * (k & 1)) * RB);
      const i16x4 lo = ds_read_tr(a), hi = ds_read_tr(a + 8 * D);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto early = [&](const char *ks) {
#pragma unroll
      for (int i = 0; i < kAhead; ++i) fq[i] = kfrag(ks, i);
    };
    auto early_v = [&](const char *vs) {
#pragma unroll
      for (int i = 0; i < kAhead; ++i) fv[i] = vfrag(vs, i);
    };
    auto mfma_run = [&](auto nq_c, auto np_c, const char *ks, const char *vs, auto pre_c, auto hook) {
      constexpr int NQ = decltype(nq_c)::value, NP = decltype(np_c)::value, N = NQ + NP;
      constexpr bool PRE = decltype(pre_c)::value;
      static_assert(!PRE || (NQ == 0 ? NP : NQ) >= kAhead, "preloaded fragments of one operand");
      auto frag = [&](int i) -> bf16x8 { return i < NQ ? kfrag(ks, i) : vfrag(vs, i - NQ); };
      bf16x8 f[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i)
        if (i < N) f[i] = PRE ? (NQ > 0 ? fq[i] : fv[i]) : frag(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const bf16x8 a = f[i % kAhead];
        if (i + kAhead < N) f[i % kAhead] = frag(i + kAhead);
        if (i < NQ) {
          s[i & 1] = mfma32(a, qf[i >> 1], i < 2 ? mref : s[i & 1]);
        } else {
          const int k = i - NQ;
          acc[k >> 2] = mfma32(a, pk[(k >> 1) & 1][k & 1], acc[k >> 2]);
        }
        hook(i);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using QK = std::integral_constant<int, 2 * KS>;
    using PV = std::integral_constant<int, 4 * DB>;
    using NONE = std::integral_constant<int, 0>;
    // Softmax phase on the scores of one tile: probabilities P (bf16, the B
    // operand of the next P.V run), the row sum l and the lazily raised
    // reference max m.
    auto softmax = [&](const It &x, int cls) {
      if (__builtin_expect(cls == TILE_DIAG, 0)) {
        // key of register r in lane half h2 is kb*32 + 8*(r/4) + 4*h2 + r%4: compare
        // its compile-time part with per-lane limits (branch-free selects)
        const int nvalid = min(BN, x.kend - x.k0);
        const int lim_c = p.causal ? my_qpos - x.k0 - x.off - 4 * h2 : BN;
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
      // (Before the first reference exists the fast path's values are discarded.)
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(s[kb][r]);
          rs += e;
          pk[kb][r >> 3][r & 7] = (__bf16)e;
        }
      if (__builtin_expect(__any(!(rs <= sum_bound)), 0)) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        // the reference max is raised only when the row max exceeds it by more
        // than 2^kTau (exact: O and l share the reference); the O rescale is rare
        const float tmax = pair_max(mx) + mu;
        if (__any(tmax > m + kTau)) {
          const float m_new = fmaxf(m, tmax);
          const float alpha = __builtin_amdgcn_exp2f(m - (m_new == -INFINITY ? 0.f : m_new));
          m = m_new;
          l *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        }
        // the scores hold s - mu; shift them to the (possibly new) reference
        const float mu_new = m == -INFINITY ? 0.f : m;
        const float d = mu_new - mu;
        mu = mu_new;
        mref = -mu;
        rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(s[kb][r] - d);
            rs += e;
            pk[kb][r >> 3][r & 7] = (__bf16)e;
          }
        sum_bound = __any(m == -INFINITY) ? -1.f : kLaneSumMax;
      }
      l += rs;
    };
    auto barrier = [] {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };

    // ---- ping-pong over the tiles.  Each wave runs C_0 S_0 C_1 S_1 ... C_n, with
    // C_j = [K.Q^T of tile j, P.V of tile j-1] on the matrix core and S_j = the
    // softmax of tile j on the vector ALU; group 1 runs one phase behind group 0,
    // and every phase ends at a workgroup barrier.  So on each SIMD one wave's
    // MFMA run meets the other wave's softmax.  In phase ph group 0 runs step
    // ph and group 1 step ph-1 of that sequence (C_j is step 2j, S_j step 2j+1).
    //
    // Tile j's K sits in K stage j%4 and is read in phases 2j and 2j+1 (its
    // first fragments at the end of phases 2j-1 and 2j); its V sits in V stage
    // j%4 and is read in phases 2j+1 to 2j+3 (its first fragments at the end of
    // S_j, phases 2j+1 and 2j+2; the P.V runs of C_j+1 in 2j+2 and 2j+3).  In
    // S_j group 0 issues all of tile j+3's K (phase 2j+1) and group 1 all of
    // tile j+3's V (phase 2j+2), into stages last read in phase 2j+1.  Past the
    // last tile the free stages are refilled with tile j, so every step has the
    // same loads in flight.  Each wave issues LO loads per S step (K0 K1 K2 |
    // K3 | K4 | ..., V0 V1 V2 | V3 | ...) and waits at the end of each C step
    // for all but those of its latest S step: at the end of C_j (phase 2j for
    // group 0, 2j+1 for group 1) K, resp. V, of tile j+1 has landed, issued
    // three phases earlier, and the barrier that follows publishes it.  Group 1
    // clears the V rows of tile j+1 past a range end in S_j (phase 2j+2),
    // published before group 0's first reads of them (phase 2j+3).
    if (n > 0) {
      // K of tile 0 has landed (pass 1: all its first loads landed before the
      // previous pass's outputs were stored, and the stores must not be waited on)
      if (pass == 0) wait_vmcnt<2 * LO>();   // K, resp. V, of tile 0
      zero_v_tail(cur, vring);
      barrier();
      early(kring);
      int cls = tile_class(cur);
      bool prev_live = false;
      // C_j: the K.Q^T run of tile j (in K stage j%4), then the P.V run of tile
      // j-1 (in V stage (j-1)%4).  The loop is unrolled over the four ring
      // stages, so that every LDS address is a per-lane offset plus an immediate.
      auto mfma_step = [&](auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        const char *ks = kring + ST * TB;
        const char *vs = vring + ((ST + NST - 1) % NST) * TB;
        __builtin_amdgcn_s_setprio(1);
        if (__builtin_expect(cls != TILE_SKIP, 1)) mfma_run(QK{}, NONE{}, ks, vs, std::true_type{}, [](int) {});
        if (__builtin_expect(prev_live, 1)) mfma_run(NONE{}, PV{}, ks, vs, std::true_type{}, [](int) {});
        __builtin_amdgcn_s_setprio(0);
        wait_vmcnt<LO>();   // all but the loads of this wave's latest S step
      };
      // S_j: this wave's part of tile j+3's K (group 0) or V (group 1) goes out
      // first, so that the loads are in flight during the softmax; group 1 then
      // clears tile j+1's V tail, and at the end each wave reads the first K
      // fragments of C_j+1's K.Q^T run and the first V fragments of its P.V run
      auto softmax_step = [&](auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        issue(ld, own_ring + ((ST + 3) % NST) * TB);
        if (__builtin_expect(cls != TILE_SKIP, 1)) softmax(cur, cls);
        prev_live = cls != TILE_SKIP;
        step2(cur, ld);
        cls = tile_class(cur);
        zero_v_tail(cur, vring + ((ST + 1) % NST) * TB);
        early(kring + ((ST + 1) % NST) * TB);
        early_v(vring + ST * TB);
      };
      using St0 = std::integral_constant<int, 0>;
      using St1 = std::integral_constant<int, 1>;
      using St2 = std::integral_constant<int, 2>;
      using St3 = std::integral_constant<int, 3>;
      static_assert(NST == 4, "the loop is unrolled over four stages");
      // tiles past the last (up to a multiple of four) are skipped by every wave
      const int n4 = (n + NST - 1) / NST * NST;
      if (grp == 1) barrier();   // group 1 runs one phase behind
      for (int j = 0; j < n4; j += NST) {
        mfma_step(St0{});
        barrier();
        softmax_step(St0{});
        barrier();
        mfma_step(St1{});
        barrier();
        softmax_step(St1{});
        barrier();
        mfma_step(St2{});
        barrier();
        softmax_step(St2{});
        barrier();
        mfma_step(St3{});
        barrier();
        softmax_step(St3{});
        barrier();
      }
      mfma_step(St0{});          // P.V of the last tile (stage (n4-1) % 4 = 3)
      barrier();
      if (grp == 0) barrier();   // group 0 waits out group 1's last phase
    }
    wait_vmcnt<0>();   // no load into LDS may outlive the pass
    __builtin_amdgcn_s_barrier();

    // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l), after pass 1's Q
    // rows and first tiles are in
    const int e_row = my_row;
    const bool e_ok = row_ok;
    if (pass == 0 && two) {
      set_pass(T - 1 - pr);
      load_q();
      start_tiles();
      wait_vmcnt<0>();
      convert_q();
    }
    const float lt = pair_sum(l);
    // bf16 rows 16-byte aligned: the lane halves swap half of their column
    // groups (permlane32_swap) so that each lane stores 8 consecutive columns:
    // half the store instructions, and each writes 32 bytes of a row per lane
    // pair instead of 16 (the store path's cost goes with the pieces touched)
    const bool o16 = !p.o_f32 && (uintptr_t)p.o % 16 == 0 && p.o_ss % 8 == 0 && p.o_sh % 8 == 0 && p.o_sb % 8 == 0;
    if (e_ok) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int64_t orow = b * p.o_sb + head * p.o_sh + (int64_t)e_row * p.o_ss;
      auto pack2 = [](float x, float y) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 w = {(__bf16)x, (__bf16)y};
        return __builtin_bit_cast(uint32_t, w);
      };
      if (o16) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; g += 2) {
            const f32x16 &a = acc[db];
            const auto x0 = __builtin_amdgcn_permlane32_swap(pack2(a[4 * g] * inv, a[4 * g + 1] * inv),
                                                             pack2(a[4 * g + 4] * inv, a[4 * g + 5] * inv), false, false);
            const auto x1 = __builtin_amdgcn_permlane32_swap(pack2(a[4 * g + 2] * inv, a[4 * g + 3] * inv),
                                                             pack2(a[4 * g + 6] * inv, a[4 * g + 7] * inv), false, false);
            *(u32x4 *)((__bf16 *)p.o + orow + db * 32 + 8 * (g + h2)) = u32x4{x0[0], x1[0], x0[1], x1[1]};
          }
      } else {
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
      }
      if (h2 == 0)
        p.lse[b * p.l_sb + head * p.l_sh + (int64_t)e_row * p.l_ss] =
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
