// Causal linear attention with a carried key/value state on bf16 MFMA tiles
// (gfx950): one device's share of LASP-style sequence parallelism.
//
// LASP summary (linnk.ai, abstract): linear attention is parallelised over the
// sequence by handing an intermediate key/value state from device to device,
// using the right-product trick and caching the intermediate KV state.  With no
// normalisation and no decay (the page prints no formula), for query head h
// and its key/value head g:
//   O_i   = sum_{j<=i} (q_i . k_j) v_j + q_i S_in,   S_out = S_in + sum_j k_j^T v_j.
// Evaluated over chunks of C = 128 rows (right product across chunks, left
// product inside one):
//   O_t = mask(Q_t K_t^T) V_t + Q_t S_{t-1},   S_t = S_{t-1} + K_t^T V_t,
// in three kernels, with the state scanned on two levels (segments of 16
// chunks), so that no per-chunk f32 state ever goes to memory:
//  - seg: per (b, g, segment) the chunks' K_t^T V_t accumulate in MFMA
//    registers (operands from LDS by ds_read_b64_tr_b16: the contraction runs
//    over the chunk's rows); before each chunk the state since the segment start
//    is stored in bf16 (the state cache), and the segment total in f32;
//  - segscan: per (b, g) the state at each segment start (S_in plus earlier
//    totals, f32, stored in bf16) and S_out;
//  - out: per (b, h, chunk), four waves of 32 query rows: S^T = K.Q^T for the
//    visible 32-key blocks (diagonal block masked), O^T += V^T.P^T with P the
//    bf16 scores, then O^T += (base + prefix)^T.Q^T for all earlier rows.
#include "internal.h"

namespace chain {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 128;   // rows per chunk
constexpr int kSeg = 16;      // chunks per segment of the two-level state scan

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: in each group of 16 lanes, lane i receives element i%4
// of the 4-element rows addressed by lanes 4e + i/4, e = 0..3.
__device__ inline i16x4 ds_read_tr(const char *p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

// Chunk swizzle of a staged row r (16-byte chunks, D/8 per row): a bijection
// over 16 consecutive rows (16-byte row reads of 16 lanes hit 16 bank groups),
// with bits 2-3 (D=128) differing over 4 aligned rows (transposing reads).
template <int D>
__device__ inline int swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Byte offset of element (row, col) of a staged tile (col a multiple of 4).
template <int D>
__device__ inline int tile_off(int row, int col) {
  return row * 2 * D + ((((col >> 3) ^ swz<D>(row))) << 4) + 2 * (col & 7);
}

// Stage R rows of D bf16 (global row stride ld elements; rows >= nrows zero).
template <int D, int R>
__device__ inline void stage_rows(char *dst, const __bf16 *src, int64_t ld, int nrows) {
  constexpr int CPR = D / 8, N = R * CPR / 256;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int c = threadIdx.x + 256 * i, row = c / CPR, ch = c % CPR;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < nrows) v = *(const u32x4 *)(src + row * ld + 8 * ch);
    *(u32x4 *)(dst + row * 2 * D + ((ch ^ swz<D>(row)) << 4)) = v;
  }
}

// A-operand fragment of T^T for a staged row-major tile T: columns c0 + lane%32,
// rows r0 + {4h..4h+3, 8+4h..8+4h+3} for lane half h (the same fragment serves as
// a B operand whose column is c0 + lane%32, with the same row order).
template <int D>
__device__ inline bf16x8 tr_frag(const char *t, int r0, int c0, int lane) {
  const int h2 = lane >> 5;
  const int trow = 4 * h2 + ((lane & 15) >> 2);
  const int tcol = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const i16x4 lo = ds_read_tr(t + tile_off<D>(r0 + trow, tcol));
  const i16x4 hi = ds_read_tr(t + tile_off<D>(r0 + trow + 8, tcol));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 16-byte row fragment: row r0 + lane%32, columns 16 ks + 8 (lane/32) .. +8.
template <int D>
__device__ inline bf16x8 row_frag(const char *t, int r0, int ks, int lane) {
  return *(const bf16x8 *)(t + tile_off<D>(r0 + (lane & 31), 16 * ks + 8 * (lane >> 5)));
}

// ---- seg: the state inside a segment of kSeg chunks, kept in MFMA accumulators
// One workgroup per (b, g, segment).  Wave w owns rows 32w.. of S^T (D = 128;
// D = 64: one 32 x 32 block per wave).  Before each chunk is added, the running
// state since the segment start is stored in bf16 (the state cache); after the
// last chunk the segment's total goes out in f32.  The next chunk's K and V are
// loaded into registers while the current one is multiplied.
template <int D>
__global__ __launch_bounds__(256) void lin_seg_kernel(const LinAttnParams p) {
  constexpr int DB = D / 32, CPR = D / 8, NL = kChunk * CPR / 256;
  __shared__ __attribute__((aligned(16))) char lds[2 * kChunk * 2 * D];
  char *ks_ = lds, *vs_ = lds + kChunk * 2 * D;
  const int T = (p.S + kChunk - 1) / kChunk, NS = (T + kSeg - 1) / kSeg;
  const int s = blockIdx.x % NS, bg = blockIdx.x / NS;
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const int t0 = s * kSeg, nt = min(kSeg, T - t0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h2 = lane >> 5, l32 = lane & 31;
  constexpr int NJ = D == 128 ? DB : 1;
  const int iv = D == 128 ? wave : wave >> 1;
  const int j0 = D == 128 ? 0 : wave & 1;
  const __bf16 *kbase = (const __bf16 *)p.k + b * p.k_sb + g * p.k_sh;
  const __bf16 *vbase = (const __bf16 *)p.v + b * p.v_sb + g * p.v_sh;
  u32x4 kr[NL], vr[NL];
  auto load = [&](int t) {
    const int r0 = t * kChunk, nrows = min(kChunk, p.S - r0);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int c = threadIdx.x + 256 * i, row = c / CPR, ch = c % CPR;
      const bool ok = row < nrows;
      kr[i] = ok ? *(const u32x4 *)(kbase + (int64_t)(r0 + row) * p.k_ss + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
      vr[i] = ok ? *(const u32x4 *)(vbase + (int64_t)(r0 + row) * p.v_ss + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int c = threadIdx.x + 256 * i, row = c / CPR, ch = c % CPR;
      const int off = row * 2 * D + ((ch ^ swz<D>(row)) << 4);
      *(u32x4 *)(ks_ + off) = kr[i];
      *(u32x4 *)(vs_ + off) = vr[i];
    }
  };
  f32x16 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x16{};
  load(t0);
  store();
  __syncthreads();
  for (int c = 0; c < nt; ++c) {
    const int t = t0 + c;
    if (c + 1 < nt) load(t + 1);
    // the state since the segment start, before chunk t: acc[j][r] is S^T at
    // d_v = 32 iv + 8(r/4) + 4h2 + r%4, d_k = 32 (j0 + j) + l32
    __bf16 *pf = p.pref + ((int64_t)bg * T + t) * D * D;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pf[(32 * iv + 8 * (r >> 2) + 4 * h2 + (r & 3)) * D + 32 * (j0 + j) + l32] = (__bf16)acc[j][r];
#pragma unroll
    for (int ks = 0; ks < kChunk / 16; ++ks) {
      const bf16x8 a = tr_frag<D>(vs_, 16 * ks, 32 * iv, lane);
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = mfma32(a, tr_frag<D>(ks_, 16 * ks, 32 * (j0 + j), lane), acc[j]);
    }
    if (c + 1 < nt) {
      __syncthreads();
      store();
      __syncthreads();
    }
  }
  float *tot = p.seg_total + ((int64_t)bg * NS + s) * D * D;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      tot[(32 * iv + 8 * (r >> 2) + 4 * h2 + (r & 3)) * D + 32 * (j0 + j) + l32] = acc[j][r];
}

// ---- segscan: the state at each segment start (bf16) and S_out ------------------
template <int D>
__global__ __launch_bounds__(256) void lin_segscan_kernel(const LinAttnParams p) {
  const int T = (p.S + kChunk - 1) / kChunk, NS = (T + kSeg - 1) / kSeg;
  constexpr int PER_HEAD = D * D / 4 / 256;   // workgroups per head
  const int bg = blockIdx.x / PER_HEAD;
  const int e = ((blockIdx.x % PER_HEAD) * 256 + threadIdx.x) * 4;   // first of 4 elements
  const int dv = e / D, dk = e % D;
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  f32x4 run = {0.f, 0.f, 0.f, 0.f};
  if (p.s_in) {
    const float *si = p.s_in + b * p.si_sb + g * p.si_sh;
#pragma unroll
    for (int u = 0; u < 4; ++u) run[u] = si[(dk + u) * p.si_sr + dv];
  }
  for (int s = 0; s < NS; ++s) {
    const int64_t o = ((int64_t)bg * NS + s) * D * D + e;
    *(bf16x4 *)(p.seg_base + o) = bf16x4{(__bf16)run[0], (__bf16)run[1], (__bf16)run[2], (__bf16)run[3]};
    run += *(const f32x4 *)(p.seg_total + o);
  }
  if (p.s_out) {
    float *so = p.s_out + b * p.so_sb + g * p.so_sh;
#pragma unroll
    for (int u = 0; u < 4; ++u) so[(dk + u) * p.so_sr + dv] = run[u];
  }
}

// ---- out: O_t = mask(Q_t K_t^T) V_t + Q_t S_{t-1} ------------------------------
template <int D>
__global__ __launch_bounds__(256) void lin_out_kernel(const LinAttnParams p) {
  constexpr int KS = D / 16, DB = D / 32, RB = 2 * D;
  __shared__ __attribute__((aligned(16))) char lds[(2 * kChunk + 2 * D) * RB];
  char *ks_ = lds, *vs_ = lds + kChunk * RB, *ss_ = lds + 2 * kChunk * RB, *sb_ = ss_ + D * RB;
  const int T = (p.S + kChunk - 1) / kChunk, NS = (T + kSeg - 1) / kSeg;
  const int t = blockIdx.x % T, bh = blockIdx.x / T;
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int g = h / (p.Hq / p.Hkv);
  const int r0 = t * kChunk, nrows = min(kChunk, p.S - r0);
  stage_rows<D, kChunk>(ks_, (const __bf16 *)p.k + b * p.k_sb + g * p.k_sh + r0 * p.k_ss, p.k_ss, nrows);
  stage_rows<D, kChunk>(vs_, (const __bf16 *)p.v + b * p.v_sb + g * p.v_sh + r0 * p.v_ss, p.v_ss, nrows);
  stage_rows<D, D>(ss_, p.pref + ((int64_t)(b * p.Hkv + g) * T + t) * D * D, D, D);
  stage_rows<D, D>(sb_, p.seg_base + ((int64_t)(b * p.Hkv + g) * NS + t / kSeg) * D * D, D, D);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h2 = lane >> 5, l32 = lane & 31;
  const int row = 32 * wave + l32;   // query row within the chunk
  const bool row_ok = row < nrows;
  bf16x8 qf[KS];
  {
    const __bf16 *qr = (const __bf16 *)p.q + b * p.q_sb + h * p.q_sh + (int64_t)(r0 + min(row, nrows - 1)) * p.q_ss + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = row_ok ? *(const bf16x8 *)(qr + 16 * ks) : bf16x8{};
  }
  __syncthreads();
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  // inside the chunk: key blocks 0..wave (the wave's queries precede later keys)
  for (int kb = 0; kb <= wave; ++kb) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = mfma32(row_frag<D>(ks_, 32 * kb, ks, lane), qf[ks], s);
    // s[r]: key 32 kb + 8(r/4) + 4h2 + r%4 of query row; mask keys past the query
    bf16x8 pk[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * kb + 8 * (r >> 2) + 4 * h2 + (r & 3);
      pk[r >> 3][r & 7] = (__bf16)(kb < wave || key <= row ? s[r] : 0.f);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        acc[db] = mfma32(tr_frag<D>(vs_, 32 * kb + 16 * hh, 32 * db, lane), pk[hh], acc[db]);
  }
  // earlier chunks through the carried state, the segment's base and the prefix
  // inside the segment: O^T += S^T . Q^T
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc[db] = mfma32(row_frag<D>(sb_, 32 * db, ks, lane), qf[ks], acc[db]);
      acc[db] = mfma32(row_frag<D>(ss_, 32 * db, ks, lane), qf[ks], acc[db]);
    }
  if (row_ok) {
    const int64_t orow = b * p.o_sb + h * p.o_sh + (int64_t)(r0 + row) * p.o_ss;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int d0 = 32 * db + 8 * gg + 4 * h2;
        const f32x4 v = {acc[db][4 * gg], acc[db][4 * gg + 1], acc[db][4 * gg + 2], acc[db][4 * gg + 3]};
        if (p.o_f32) *(f32x4 *)((float *)p.o + orow + d0) = v;
        else *(bf16x4 *)((__bf16 *)p.o + orow + d0) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
      }
  }
}

template <int D>
hipError_t launch_d(const LinAttnParams &p, hipStream_t s) {
  const int T = (p.S + kChunk - 1) / kChunk, NS = (T + kSeg - 1) / kSeg;
  hipLaunchKernelGGL(lin_seg_kernel<D>, dim3(p.B * p.Hkv * NS), dim3(256), 0, s, p);
  hipLaunchKernelGGL(lin_segscan_kernel<D>, dim3(p.B * p.Hkv * (D * D / 1024)), dim3(256), 0, s, p);
  hipLaunchKernelGGL(lin_out_kernel<D>, dim3(p.B * p.Hq * T), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// Workspace: [in-segment prefix per chunk, bf16 | segment totals, f32 | segment bases, bf16].
void linear_attn_workspace_layout(int64_t B, int64_t Hkv, int64_t S, int64_t D, size_t off[4]) {
  const int64_t T = (S + kChunk - 1) / kChunk, NS = (T + kSeg - 1) / kSeg;
  const size_t per_chunk = (size_t)B * Hkv * T * D * D, per_seg = (size_t)B * Hkv * NS * D * D;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  off[0] = 0;
  off[1] = off[0] + up(per_chunk * 2);
  off[2] = off[1] + up(per_seg * 4);
  off[3] = off[2] + up(per_seg * 2);
}

size_t linear_attn_workspace_bytes(int64_t B, int64_t Hkv, int64_t S, int64_t D) {
  size_t off[4];
  linear_attn_workspace_layout(B, Hkv, S, D, off);
  return off[3];
}

hipError_t launch_linear_attn(const LinAttnParams &p, int D, hipStream_t s) {
  if (p.B == 0 || p.Hkv == 0) return hipSuccess;
  if (p.S == 0) {
    // no rows: S_out = S_in (or 0); the scan over zero segments writes exactly that
    if (!p.s_out) return hipSuccess;
    if (D == 64) hipLaunchKernelGGL(lin_segscan_kernel<64>, dim3(p.B * p.Hkv * 4), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(lin_segscan_kernel<128>, dim3(p.B * p.Hkv * 16), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  return D == 64 ? launch_d<64>(p, s) : launch_d<128>(p, s);
}

}  // namespace chain
