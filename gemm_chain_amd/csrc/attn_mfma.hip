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
// Eight waves per workgroup (two per SIMD) share each staged 64-key K/V tile;
// tiles are double-buffered in LDS, and the global loads run two tiles ahead
// (two register sets: tile i+2 is fetched while tile i is computed and tile
// i+1, fetched one step earlier, is written to the free LDS buffer).  LDS pitches are chosen for conflict-free 16-byte
// K reads (D+8) and conflict-free transposing V reads (D+32).  Inside each MFMA
// run the LDS fragments are read kAhead MFMAs ahead of use (pinned with
// scheduling barriers) and the wave raises its issue priority, so the other
// wave on the SIMD fills the VALU (softmax) while this one feeds the matrix
// core.  The reference max is raised only when a row's max grows past it by
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

constexpr int BN = 64;          // keys per tile
constexpr float kTau = 8.0f;    // lazy rescale threshold (base-2 exponent)
constexpr int kAhead = 4;       // LDS fragments in flight ahead of their MFMA

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: in each group of 16 lanes, lane i receives element i%4
// of the 4-element rows addressed by lanes 4e + i/4, e = 0..3.
__device__ inline i16x4 ds_read_tr(const __bf16 *p) {
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

template <int D, int NW, int WH>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(2)))
void attn_mfma_bf16_kernel(const AttnParams p) {
  constexpr int WQ = NW / WH;               // 32-row query blocks per head
  constexpr int ROWS = 32 * WQ;             // query positions per tile
  constexpr int KS = D / 16;                // k-steps of K.Q^T
  constexpr int DB = D / 32;                // 32-wide blocks of O^T
  constexpr int LDK = D + 8;                // K pitch: conflict-free 16-byte reads
  constexpr int LDV = D + 32;               // V pitch: conflict-free transposing reads
  constexpr int CPR = D / 8;                // 16-byte chunks per key row
  constexpr int LOADS = BN * CPR / (NW * 64);
  constexpr int BUF = BN * (LDK + LDV);
  static_assert(LOADS * NW * 64 == BN * CPR, "tile must split evenly over the workgroup");
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
    struct Tl { int ri, k0; bool valid; };
    auto first_tile = [&]() -> Tl {
      for (int r = 0; r < p.kr.n; ++r)
        if (range_live(r)) return Tl{r, p.kr.beg[r], true};
      return Tl{0, 0, false};
    };
    auto next_tile = [&](Tl x) -> Tl {
      if (!x.valid) return x;
      int r = x.ri, k = x.k0;
      return advance(r, k) ? Tl{r, k, true} : Tl{0, 0, false};
    };
    // global loads run two tiles ahead: tile j+2 is fetched into one register
    // set while the set holding tile j+1 is written to LDS after tile j
    uint4 kA[LOADS], vA[LOADS], kB[LOADS], vB[LOADS];
    auto gload2 = [&](uint4 (&kr)[LOADS], uint4 (&vr)[LOADS], const Tl &x) {
      const int kend = p.kr.end[x.ri];
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int cidx = tid + i * NW * 64;
        const int r = cidx / CPR, c8 = cidx % CPR;
        const int key = x.k0 + r;
        if (key < kend) {
          kr[i] = *(const uint4 *)(kbase + (int64_t)key * p.k_ss + c8 * 8);
          vr[i] = *(const uint4 *)(vbase + (int64_t)key * p.v_ss + c8 * 8);
        } else {
          kr[i] = make_uint4(0, 0, 0, 0);
          vr[i] = make_uint4(0, 0, 0, 0);
        }
      }
    };
    auto swrite2 = [&](const uint4 (&kr)[LOADS], const uint4 (&vr)[LOADS], int buf) {
      __bf16 *ks = smem + buf * BUF;
      __bf16 *vs = ks + BN * LDK;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int cidx = tid + i * NW * 64;
        const int r = cidx / CPR, c8 = cidx % CPR;
        *(uint4 *)(ks + r * LDK + c8 * 8) = kr[i];
        *(uint4 *)(vs + r * LDV + c8 * 8) = vr[i];
      }
    };
    auto compute = [&](const int ri, const int k0, const int buf) {
      // ---- compute on the staged tile
      const int off = p.kr.pos_off[ri];
      const int nvalid = min(BN, p.kr.end[ri] - k0);
      const int cls = classify_tile(p.causal, w_qmin, w_qmax, k0 + off, k0 + nvalid - 1 + off, nvalid < BN);
      if (wave_rows && cls != TILE_SKIP) {
        const __bf16 *ks = smem + buf * BUF;
        const __bf16 *vs = ks + BN * LDK;
        f32x16 s[2] = {f32x16{}, f32x16{}};
        __builtin_amdgcn_s_setprio(1);
        {
          constexpr int N = 2 * KS;
          auto addr = [&](int i) { return ks + ((i & 1) * 32 + l32) * LDK + (i >> 1) * 16 + 8 * h2; };
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
        float rs = 0.f;
        bf16x8 pk[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -m_use));
            rs += e;
            pk[kb][r >> 3][r & 7] = (__bf16)e;
          }
        l += rs;
        // O^T += V^T . P^T
        const int trow = 4 * h2 + ((lane & 15) >> 2);
        const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        __builtin_amdgcn_s_setprio(1);
        {
          constexpr int N = 4 * DB;
          auto addr = [&](int i) {
            const int db = i >> 2, kb = (i >> 1) & 1, hh = i & 1;
            return vs + (kb * 32 + 16 * hh + trow) * LDV + db * 32 + tcol;
          };
          i16x4 vlo[kAhead], vhi[kAhead];
#pragma unroll
          for (int i = 0; i < kAhead; ++i) {
            vlo[i] = ds_read_tr(addr(i));
            vhi[i] = ds_read_tr(addr(i) + 8 * LDV);
          }
#pragma unroll
          for (int i = 0; i < N; ++i) {
            const i16x8 a16 = __builtin_shufflevector(vlo[i % kAhead], vhi[i % kAhead], 0, 1, 2, 3, 4, 5, 6, 7);
            if (i + kAhead < N) {
              vlo[i % kAhead] = ds_read_tr(addr(i + kAhead));
              vhi[i % kAhead] = ds_read_tr(addr(i + kAhead) + 8 * LDV);
            }
            acc[i >> 2] = mfma32(__builtin_bit_cast(bf16x8, a16), pk[(i >> 1) & 1][i & 1], acc[i >> 2]);
        __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };

    Tl w0 = first_tile(), w1 = next_tile(w0), w2 = next_tile(w1);
    if (w0.valid) {
      gload2(kA, vA, w0);
      swrite2(kA, vA, 0);
    }
    if (w1.valid) gload2(kB, vB, w1);
    __syncthreads();
    int j = 0;
    // x: register set holding w1 (written to LDS after this tile); y: set for w2
    auto step = [&](uint4 (&kx)[LOADS], uint4 (&vx)[LOADS], uint4 (&ky)[LOADS], uint4 (&vy)[LOADS]) {
      const int buf = j & 1;
      if (w2.valid) gload2(ky, vy, w2);
      compute(w0.ri, w0.k0, buf);
      if (w1.valid) swrite2(kx, vx, buf ^ 1);
      __syncthreads();
      w0 = w1;
      w1 = w2;
      w2 = next_tile(w2);
      ++j;
    };
    while (w0.valid) {
      step(kB, vB, kA, vA);
      if (!w0.valid) break;
      step(kA, vA, kB, vB);
    }

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

template <int D, int NW, int WH>
hipError_t launch(const AttnParams &p, hipStream_t s) {
  constexpr int ROWS = 32 * (NW / WH);
  const int T = (p.Sq + ROWS - 1) / ROWS;
  const int items = p.B * (p.Hq / WH) * ((T + 1) / 2);
  hipLaunchKernelGGL((attn_mfma_bf16_kernel<D, NW, WH>), dim3(items), dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams &p, hipStream_t s) {
  const int group = p.Hq / p.Hkv;
  if (group % 4 == 0) return launch<D, 8, 4>(p, s);
  if (group % 2 == 0) return launch<D, 8, 2>(p, s);
  return launch<D, 8, 1>(p, s);
}

}  // namespace

hipError_t launch_attn_mfma_bf16(const AttnParams &p, int D, hipStream_t s) {
  return D == 64 ? launch_d<64>(p, s) : launch_d<128>(p, s);
}

}  // namespace chain
