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
// Three kernels, no atomics (every output element is written once, so reruns
// give identical bits):
//  - rowdot: D_i for every query row into the workspace.
//  - dq: a workgroup of four waves (one per SIMD) takes 32-row query blocks of
//    WH heads of one key/value head and walks the visible 64-key tiles, staged
//    in LDS.  Per tile and wave: S^T = K.Q^T and dP^T = V.dO^T (Q and dO
//    fragments stay in registers; each lane owns one query, as in the
//    forward), dS^T = P^T * (dP^T - D) in registers, then dQ^T += K^T.dS^T with
//    K^T read by ds_read_b64_tr_b16 in the key order the dS^T accumulator holds.
//  - dkdv: a workgroup of four waves takes 128 keys of one key/value head (32
//    per wave, their K and V fragments in registers) and walks every visible
//    32-row query tile of every query head of the group, staged in LDS with its
//    log-sum-exp and D values.  Per tile and wave: S = Q.K^T and dP = dO.V^T,
//    P and dS, then dV^T += dO^T.P and dK^T += Q^T.dS with dO^T and Q^T read
//    transposed.
// Query tiles (dq) and key blocks (dkdv) are taken in pairs t, T-1-t so causal
// work per workgroup is even, and workgroups of one key/value head share an XCD.
#include "internal.h"

namespace chain {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: in each group of 16 lanes, lane i receives element i%4
// of the 4-element rows addressed by lanes 4e + i/4, e = 0..3.
__device__ inline i16x4 ds_read_tr(const __bf16 *p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

// A-operand fragment of T^T for a row-major tile T (pitch `pitch`): columns
// c0 + lane%32 of T, rows r0 + {4h..4h+3, 8+4h..8+4h+3} for lane half h -- the
// row order in which a 32x32 accumulator packed by pack_half() holds them.
__device__ inline bf16x8 tr_frag(const __bf16 *t, int pitch, int r0, int c0, int trow, int tcol) {
  const __bf16 *a = t + (r0 + trow) * pitch + c0 + tcol;
  const i16x4 lo = ds_read_tr(a);
  const i16x4 hi = ds_read_tr(a + 8 * pitch);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Rows 16*hh .. 16*hh + 15 of a 32x32 accumulator (registers 8*hh .. 8*hh + 7),
// rounded to bf16: the B operand of a product that contracts over those rows.
__device__ inline bf16x8 pack_half(const f32x16 &c, int hh) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)c[8 * hh + j];
  return r;
}

// ---- D_i = sum_d dO_id O_id ------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void rowdot_kernel(const AttnBwdParams p) {
  constexpr int CPR = D / 8, RPB = 256 / CPR;
  const int64_t rows = (int64_t)p.B * p.Hq * p.S;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / CPR;
  const int c = threadIdx.x % CPR;
  float acc = 0.f;
  if (row < rows) {
    const int s = (int)(row % p.S), h = (int)((row / p.S) % p.Hq), b = (int)(row / ((int64_t)p.S * p.Hq));
    const bf16x8 o = *(const bf16x8 *)((const __bf16 *)p.o + b * p.o_sb + h * p.o_sh + (int64_t)s * p.o_ss + 8 * c);
    const bf16x8 g = *(const bf16x8 *)((const __bf16 *)p.dout + b * p.do_sb + h * p.do_sh + (int64_t)s * p.do_ss + 8 * c);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf((float)o[j], (float)g[j], acc);
  }
#pragma unroll
  for (int w = CPR / 2; w > 0; w >>= 1) acc += __shfl_xor(acc, w, CPR);
  if (row < rows && c == 0) p.drow[row] = acc;
}

// ---- dQ ----------------------------------------------------------------------
template <int D, int WH>
__device__ __forceinline__ void dq_body(const AttnBwdParams &p) {
  constexpr int NW = 4, WQ = NW / WH, ROWS = 32 * WQ;
  constexpr int KS = D / 16, DB = D / 32, BN = 64;
  constexpr int LDT = D + 8;                        // staged K and V pitch
  constexpr int CPR = D / 8;
  constexpr int LOADS = BN * CPR / (NW * 64);
  __shared__ __attribute__((aligned(16))) __bf16 smem[2][2][BN * LDT];   // [buffer][K, V]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h2 = lane >> 5, l32 = lane & 31;
  const int trow = 4 * h2 + ((lane & 15) >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

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
  const __bf16 *kbase = (const __bf16 *)p.k + b * p.k_sb + kvh * p.k_sh;
  const __bf16 *vbase = (const __bf16 *)p.v + b * p.v_sb + kvh * p.v_sh;
  const float c = p.scale_log2;

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
    {
      const __bf16 *qr = (const __bf16 *)p.q + b * p.q_sb + head * p.q_sh + (int64_t)rr * p.q_ss + 8 * h2;
      const __bf16 *gr = (const __bf16 *)p.dout + b * p.do_sb + head * p.do_sh + (int64_t)rr * p.do_ss + 8 * h2;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = row_ok ? *(const bf16x8 *)(qr + 16 * ks) : bf16x8{};
        dof[ks] = row_ok ? *(const bf16x8 *)(gr + 16 * ks) : bf16x8{};
      }
    }
    const float lse = p.lse[b * p.l_sb + head * p.l_sh + (int64_t)rr * p.l_ss];
    // no visible key (LSE = -inf): every probability is 0
    const float lse2 = (row_ok && lse != -INFINITY) ? lse * kLog2e : INFINITY;
    const float drow = p.drow[((int64_t)b * p.Hq + head) * p.S + rr];
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

    const int nkt = p.causal ? wg_qmax / BN + 1 : (p.S + BN - 1) / BN;
    uint4 kr[LOADS], vr[LOADS];
    auto gload = [&](int kt) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int ci = tid + i * NW * 64;
        const int key = kt * BN + ci / CPR, c8 = ci % CPR;
        if (key < p.S) {
          kr[i] = *(const uint4 *)(kbase + (int64_t)key * p.k_ss + c8 * 8);
          vr[i] = *(const uint4 *)(vbase + (int64_t)key * p.v_ss + c8 * 8);
        } else {
          kr[i] = make_uint4(0, 0, 0, 0);
          vr[i] = make_uint4(0, 0, 0, 0);
        }
      }
    };
    auto swrite = [&](int buf) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int ci = tid + i * NW * 64;
        *(uint4 *)(&smem[buf][0][(ci / CPR) * LDT + (ci % CPR) * 8]) = kr[i];
        *(uint4 *)(&smem[buf][1][(ci / CPR) * LDT + (ci % CPR) * 8]) = vr[i];
      }
    };

    gload(0);
    swrite(0);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nkt) gload(kt + 1);
      const int k0 = kt * BN;
      const bool live = wave_rows && (!p.causal || k0 <= w_qmax);
      if (live) {
        const __bf16 *ks = smem[buf][0];
        const __bf16 *vs = smem[buf][1];
        f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int i = 0; i < 2 * KS; ++i) {
          const int off = ((i & 1) * 32 + l32) * LDT + (i >> 1) * 16 + 8 * h2;
          s[i & 1] = mfma32(*(const bf16x8 *)(ks + off), qf[i >> 1], s[i & 1]);
          dp[i & 1] = mfma32(*(const bf16x8 *)(vs + off), dof[i >> 1], dp[i & 1]);
        }
        // lane (h2, l32) holds key k0 + kb*32 + 8*(r/4) + 4*h2 + r%4 of query my_row
        f32x16 ds[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
            const bool vis = key < p.S && (!p.causal || key <= my_row);
            const float pr_ = vis ? __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -lse2)) : 0.f;
            ds[kb][r] = pr_ * (dp[kb][r] - drow);
          }
        // dQ^T += K^T . dS^T
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
              acc[db] = mfma32(tr_frag(ks, LDT, kb * 32 + 16 * hh, db * 32, trow, tcol), pack_half(ds[kb], hh), acc[db]);
      }
      // buf ^ 1 was last read before the previous step's barrier
      if (kt + 1 < nkt) {
        swrite(buf ^ 1);
        __syncthreads();
      }
    }
    __syncthreads();

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
  constexpr int NW = 4, KB = 32 * NW, QT = 32;
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int LDT = D + 8;                        // staged Q and dO pitch
  constexpr int CPR = D / 8;
  constexpr int LOADS = QT * CPR / (NW * 64);
  __shared__ __attribute__((aligned(16))) __bf16 smem[2][2][QT * LDT];   // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float rowv[2][2][QT];          // [buffer][LSE*log2e, D]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h2 = lane >> 5, l32 = lane & 31;
  const int trow = 4 * h2 + ((lane & 15) >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  const int group = p.Hq / p.Hkv;
  const int NB = (p.S + KB - 1) / KB;
  const int n_pairs = (NB + 1) / 2;
  const int item = xcd_remap(blockIdx.x, p.B * p.Hkv * n_pairs);
  const int pr = item % n_pairs;
  const int kvh = (item / n_pairs) % p.Hkv;
  const int b = item / (n_pairs * p.Hkv);
  const float c = p.scale_log2;
  const int nqt = (p.S + QT - 1) / QT;

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
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kf[ks] = key_ok ? *(const bf16x8 *)(kr + 16 * ks) : bf16x8{};
        vf[ks] = key_ok ? *(const bf16x8 *)(vr + 16 * ks) : bf16x8{};
      }
    }
    f32x16 dva[DB], dka[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dva[db] = f32x16{}, dka[db] = f32x16{};

    // (head of the group, query tile): the tiles that can see a key of the block
    const int t0 = p.causal ? kb0 / QT : 0;
    const int per_head = nqt - t0;
    const int steps = group * per_head;
    uint4 qr[LOADS], gr[LOADS];
    float rv = 0.f;
    auto gload = [&](int st) {
      const int head = kvh * group + st / per_head;
      const int q0 = (t0 + st % per_head) * QT;
      const __bf16 *qb = (const __bf16 *)p.q + b * p.q_sb + head * p.q_sh;
      const __bf16 *gb = (const __bf16 *)p.dout + b * p.do_sb + head * p.do_sh;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int ci = tid + i * NW * 64;
        const int row = q0 + ci / CPR, c8 = ci % CPR;
        if (row < p.S) {
          qr[i] = *(const uint4 *)(qb + (int64_t)row * p.q_ss + c8 * 8);
          gr[i] = *(const uint4 *)(gb + (int64_t)row * p.do_ss + c8 * 8);
        } else {
          qr[i] = make_uint4(0, 0, 0, 0);
          gr[i] = make_uint4(0, 0, 0, 0);
        }
      }
      if (tid < 2 * QT) {
        const int row = q0 + (tid % QT);
        if (row >= p.S) {
          rv = tid < QT ? INFINITY : 0.f;   // padding rows: probability 0
        } else if (tid < QT) {
          const float lse = p.lse[b * p.l_sb + head * p.l_sh + (int64_t)row * p.l_ss];
          rv = lse == -INFINITY ? INFINITY : lse * kLog2e;
        } else {
          rv = p.drow[((int64_t)b * p.Hq + head) * p.S + row];
        }
      }
    };
    auto swrite = [&](int buf) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int ci = tid + i * NW * 64;
        *(uint4 *)(&smem[buf][0][(ci / CPR) * LDT + (ci % CPR) * 8]) = qr[i];
        *(uint4 *)(&smem[buf][1][(ci / CPR) * LDT + (ci % CPR) * 8]) = gr[i];
      }
      if (tid < 2 * QT) rowv[buf][tid / QT][tid % QT] = rv;
    };

    if (steps > 0) {
      gload(0);
      swrite(0);
    }
    __syncthreads();
    for (int st = 0; st < steps; ++st) {
      const int buf = st & 1;
      if (st + 1 < steps) gload(st + 1);
      const int q0 = (t0 + st % per_head) * QT;
      const bool live = wave_keys && (!p.causal || q0 + QT - 1 >= kw0);
      if (live) {
        const __bf16 *qs = smem[buf][0];
        const __bf16 *gs = smem[buf][1];
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int off = l32 * LDT + ks * 16 + 8 * h2;
          s = mfma32(*(const bf16x8 *)(qs + off), kf[ks], s);
          dp = mfma32(*(const bf16x8 *)(gs + off), vf[ks], dp);
        }
        // lane (h2, l32) holds query q0 + 8*(r/4) + 4*h2 + r%4 of key my_key
        f32x16 pm, dsm;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = *(const f32x4 *)(&rowv[buf][0][8 * g + 4 * h2]);
          const f32x4 d4 = *(const f32x4 *)(&rowv[buf][1][8 * g + 4 * h2]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            const int q = q0 + 8 * g + 4 * h2 + e;
            const bool vis = key_ok && (!p.causal || my_key <= q);
            const float pr_ = vis ? __builtin_amdgcn_exp2f(fmaf(s[r], c, -l4[e])) : 0.f;
            pm[r] = pr_;
            dsm[r] = pr_ * (dp[r] - d4[e]);
          }
        }
        // dV^T += dO^T . P and dK^T += Q^T . dS (contraction over the tile's queries)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            dva[db] = mfma32(tr_frag(gs, LDT, 16 * hh, db * 32, trow, tcol), pack_half(pm, hh), dva[db]);
            dka[db] = mfma32(tr_frag(qs, LDT, 16 * hh, db * 32, trow, tcol), pack_half(dsm, hh), dka[db]);
          }
      }
      // buf ^ 1 was last read before the previous step's barrier
      if (st + 1 < steps) {
        swrite(buf ^ 1);
        __syncthreads();
      }
    }
    __syncthreads();

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
  __global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))          \
  void attn_bwd_dq_kernel_d##D##_g1(const AttnBwdParams p) { dq_body<D, 1>(p); }                        \
  __global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))          \
  void attn_bwd_dq_kernel_d##D##_g2(const AttnBwdParams p) { dq_body<D, 2>(p); }                        \
  __global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))          \
  void attn_bwd_dq_kernel_d##D##_g4(const AttnBwdParams p) { dq_body<D, 4>(p); }                        \
  __global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))          \
  void attn_bwd_dkdv_kernel_d##D(const AttnBwdParams p) { dkdv_body<D>(p); }
CHAIN_BWD_KERNELS(64)
CHAIN_BWD_KERNELS(128)
#undef CHAIN_BWD_KERNELS

template <int D>
hipError_t launch_d(const AttnBwdParams &p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.Hq * p.S;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL(rowdot_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, p);
  const int group = p.Hq / p.Hkv;
  const int wh = group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
  const int rows_t = 32 * (4 / wh);
  const int T = (p.S + rows_t - 1) / rows_t;
  const dim3 gq(p.B * (p.Hq / wh) * ((T + 1) / 2));
  if (wh == 4) hipLaunchKernelGGL((D == 64 ? attn_bwd_dq_kernel_d64_g4 : attn_bwd_dq_kernel_d128_g4), gq, dim3(256), 0, s, p);
  else if (wh == 2) hipLaunchKernelGGL((D == 64 ? attn_bwd_dq_kernel_d64_g2 : attn_bwd_dq_kernel_d128_g2), gq, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((D == 64 ? attn_bwd_dq_kernel_d64_g1 : attn_bwd_dq_kernel_d128_g1), gq, dim3(256), 0, s, p);
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
