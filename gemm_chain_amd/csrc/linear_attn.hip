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
// in two passes over the sequence with a short scan between them; no per-chunk
// state ever goes to memory:
//  - sub: per (b, g, sub-segment of consecutive chunks) the sum of the chunks'
//    K_t^T V_t, accumulated in MFMA registers (both operands from LDS by
//    ds_read_b64_tr_b16: the contraction runs over the chunk's rows), stored in f32;
//  - scan: per (b, g) the state at the start of each segment (a run of
//    consecutive sub-segments; S_in plus the earlier sums, f32) and S_out;
//  - out: per (b, h, segment) one workgroup walks the segment's rows in order
//    with the state in f32 MFMA registers, in pieces of 64 rows (D = 128, so
//    that two workgroups fit per CU) or 128 rows (D = 64).  Per piece, each wave
//    takes 32 query rows and a share of the d_v columns: S^T = K.Q^T for the
//    visible 32-key blocks (the diagonal block masked), O^T += V^T.P^T with P
//    the bf16 scores, and O^T += S^T.Q^T with the state before the piece rounded
//    to bf16 once, through LDS; then the state takes the piece's K^T V.  The
//    next piece's Q, K and V are loaded into registers while the current one is
//    computed, and its O is stored after the next piece is staged.
// Sub-segments are sized so that the first pass fills the chip; a segment is as
// many sub-segments as the key/value head has query heads (at most), so that
// the out pass has about as many workgroups again.
#include "internal.h"

#include <algorithm>

namespace chain {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 128;   // rows per chunk (the unit of the sub-segments)
constexpr int kFill = 512;    // workgroups each pass aims at (two per compute unit)
constexpr int kSubFill = 256; // workgroups of the first pass (one per compute unit)

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

// R rows of D bf16 in registers (16 bytes per thread and load), in the order a
// staged tile is written; rows >= nrows are staged as zero.
template <int D, int R = kChunk>
struct ChunkRegs {
  static constexpr int CPR = D / 8, NL = R * CPR / 256;
  u32x4 r[NL];
  int n;
  // rows past the end read the last row (every load stays inside the tensor) and
  // are written as zero
  __device__ inline void load(const __bf16 *src, int64_t ld, int nrows) {
    n = nrows;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int c = threadIdx.x + 256 * i, row = c / CPR, ch = c % CPR;
      r[i] = *(const u32x4 *)(src + min(row, nrows - 1) * ld + 8 * ch);
    }
  }
  __device__ inline void store(char *dst) const {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int c = threadIdx.x + 256 * i, row = c / CPR, ch = c % CPR;
      *(u32x4 *)(dst + row * 2 * D + ((ch ^ swz<D>(row)) << 4)) = row < n ? r[i] : u32x4{0u, 0u, 0u, 0u};
    }
  }
};

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

// ---- sub: the sum of K_t^T V_t over each sub-segment's chunks ---------------
// One workgroup per (b, g, run of sub_per_wg consecutive sub-segments).  D = 128:
// wave w owns the d_k rows 32w.. of S and all d_v columns; D = 64: one 32 x 32
// block per wave.  The next chunk's K and V are loaded into registers while the
// current one is multiplied; each sub-segment's sum goes out as it completes.
template <int D>
__global__ __launch_bounds__(256) void lin_sub_kernel(const LinAttnParams p) {
  constexpr int NJ = D == 128 ? D / 32 : 1;
  __shared__ __attribute__((aligned(16))) char lds[2 * kChunk * 2 * D];
  char *ks_ = lds, *vs_ = lds + kChunk * 2 * D;
  const int T = (p.S + kChunk - 1) / kChunk;
  const int nwg = (p.n_sub + p.sub_per_wg - 1) / p.sub_per_wg;   // workgroups per head
  const int w = blockIdx.x % nwg, bg = blockIdx.x / nwg;
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const int s0 = w * p.sub_per_wg;
  const int t0 = s0 * p.sub_len, tend = min(min(s0 + p.sub_per_wg, p.n_sub) * p.sub_len, T);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h2 = lane >> 5, l32 = lane & 31;
  const int iv = D == 128 ? wave : wave >> 1;   // d_k block
  const int j0 = D == 128 ? 0 : wave & 1;       // first d_v block
  const __bf16 *kbase = (const __bf16 *)p.k + b * p.k_sb + g * p.k_sh;
  const __bf16 *vbase = (const __bf16 *)p.v + b * p.v_sb + g * p.v_sh;
  ChunkRegs<D> kr, vr;
  auto load = [&](int t) {
    const int r0 = t * kChunk, n = min(kChunk, p.S - r0);
    kr.load(kbase + (int64_t)r0 * p.k_ss, p.k_ss, n);
    vr.load(vbase + (int64_t)r0 * p.v_ss, p.v_ss, n);
  };
  f32x16 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x16{};
  load(t0);
  kr.store(ks_);
  vr.store(vs_);
  __syncthreads();
  for (int t = t0; t < tend; ++t) {
    const bool more = t + 1 < tend;
    if (more) load(t + 1);
#pragma unroll
    for (int ks = 0; ks < kChunk / 16; ++ks) {
      const bf16x8 a = tr_frag<D>(ks_, 16 * ks, 32 * iv, lane);
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = mfma32(a, tr_frag<D>(vs_, 16 * ks, 32 * (j0 + j), lane), acc[j]);
    }
    if ((t + 1) % p.sub_len == 0 || !more) {
      // acc[j][r] is S at d_k = 32 iv + 8(r/4) + 4h2 + r%4, d_v = 32 (j0 + j) + l32
      float *tot = p.sub_total + ((int64_t)bg * p.n_sub + t / p.sub_len) * D * D;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          tot[(32 * iv + 8 * (r >> 2) + 4 * h2 + (r & 3)) * D + 32 * (j0 + j) + l32] = acc[j][r];
        acc[j] = f32x16{};
      }
    }
    if (more) {
      __syncthreads();
      kr.store(ks_);
      vr.store(vs_);
      __syncthreads();
    }
  }
}

// ---- scan: the state at each segment start (f32) and S_out --------------------
template <int D>
__global__ __launch_bounds__(256) void lin_scan_kernel(const LinAttnParams p) {
  constexpr int PER_HEAD = D * D / 4 / 256;   // workgroups per head
  const int bg = blockIdx.x / PER_HEAD;
  const int e = ((blockIdx.x % PER_HEAD) * 256 + threadIdx.x) * 4;   // first of 4 elements
  const int dk = e / D, dv = e % D;
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  f32x4 run = {0.f, 0.f, 0.f, 0.f};
  if (p.s_in) {
    const float *si = p.s_in + b * p.si_sb + g * p.si_sh + dk * p.si_sr + dv;
#pragma unroll
    for (int u = 0; u < 4; ++u) run[u] = si[u];
  }
  const int64_t head = (int64_t)bg * p.n_sub * D * D + e;
  for (int i = 0; i < p.n_seg; ++i) {
    *(f32x4 *)(p.seg_base + head + (int64_t)i * D * D) = run;
    const int j1 = min((i + 1) * p.seg_subs, p.n_sub);
    for (int j = i * p.seg_subs; j < j1; ++j) run += *(const f32x4 *)(p.sub_total + head + (int64_t)j * D * D);
  }
  if (p.s_out) {
    float *so = p.s_out + b * p.so_sb + g * p.so_sh + dk * p.so_sr + dv;
#pragma unroll
    for (int u = 0; u < 4; ++u) so[u] = run[u];
  }
}

// ---- out: O_t = mask(Q_t K_t^T) V_t + Q_t S_{t-1}, one segment per workgroup ---
// The segment is walked in pieces of CR rows (CR = 64 at D = 128, so that two
// workgroups fit per CU; 128 at D = 64).  Wave w takes the 32 query rows of block
// w % (CR/32) and DBW = D/32 / (4 / (CR/32)) of the d_v blocks.
template <int D>
constexpr int out_rows() { return D == 128 ? 64 : 128; }

// O^T of 32 query rows (columns l32), d_v blocks db0.. of the accumulators, to memory.
template <int D, int DBW>
__device__ inline void store_o(const LinAttnParams &p, const f32x16 (&acc)[DBW], int db0, int64_t orow, int h2) {
  if (p.o_f32) {
#pragma unroll
    for (int i = 0; i < DBW; ++i)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        *(f32x4 *)((float *)p.o + orow + 32 * (db0 + i) + 8 * gg + 4 * h2) =
            f32x4{acc[i][4 * gg], acc[i][4 * gg + 1], acc[i][4 * gg + 2], acc[i][4 * gg + 3]};
  } else {
#pragma unroll
    for (int i = 0; i < DBW; ++i)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        *(bf16x4 *)((__bf16 *)p.o + orow + 32 * (db0 + i) + 8 * gg + 4 * h2) =
            bf16x4{(__bf16)acc[i][4 * gg], (__bf16)acc[i][4 * gg + 1], (__bf16)acc[i][4 * gg + 2],
                   (__bf16)acc[i][4 * gg + 3]};
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void lin_out_kernel(const LinAttnParams p) {
  constexpr int CR = out_rows<D>(), NQB = CR / 32, DBW = D / 32 / (4 / NQB);
  constexpr int KS = D / 16, RB = 2 * D, NJ = D == 128 ? D / 32 : 1;
  __shared__ __attribute__((aligned(16))) char lds[(3 * CR + D) * RB];
  char *ks_ = lds, *vs_ = lds + CR * RB, *qs_ = lds + 2 * CR * RB, *ss_ = lds + 3 * CR * RB;
  const int sg = blockIdx.x % p.n_seg, bh = blockIdx.x / p.n_seg;
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int g = h / (p.Hq / p.Hkv);
  const int seg_len = p.seg_subs * p.sub_len;   // in kChunk-row chunks
  const int t0 = sg * seg_len;
  const int row_begin = t0 * kChunk;
  const int row_end = (int)std::min<int64_t>((int64_t)(t0 + seg_len) * kChunk, p.S);
  const int np = (row_end - row_begin + CR - 1) / CR;   // pieces of CR rows
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h2 = lane >> 5, l32 = lane & 31;
  const int qb = wave % NQB;                    // the wave's query block
  const int db0 = (wave / NQB) * DBW;           // its first d_v block of O
  const int iv = D == 128 ? wave : wave >> 1;   // its d_k block of the state
  const int j0 = D == 128 ? 0 : wave & 1;       // its first d_v block of the state
  const int row = 32 * qb + l32;                // query row within the piece
  const __bf16 *qbase = (const __bf16 *)p.q + b * p.q_sb + h * p.q_sh;
  const __bf16 *kbase = (const __bf16 *)p.k + b * p.k_sb + g * p.k_sh;
  const __bf16 *vbase = (const __bf16 *)p.v + b * p.v_sb + g * p.v_sh;
  ChunkRegs<D, CR> kr, vr, qr;
  auto load = [&](int r0) {
    const int n = min(CR, p.S - r0);
    kr.load(kbase + (int64_t)r0 * p.k_ss, p.k_ss, n);
    vr.load(vbase + (int64_t)r0 * p.v_ss, p.v_ss, n);
    qr.load(qbase + (int64_t)r0 * p.q_ss, p.q_ss, n);
  };
  // the state: st[j][r] is S at d_k = 32 iv + 8(r/4) + 4h2 + r%4, d_v = 32 (j0 + j) + l32
  f32x16 st[NJ];
  {
    const float *base = p.seg_base + ((int64_t)(b * p.Hkv + g) * p.n_sub + sg) * D * D;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        st[j][r] = base[(32 * iv + 8 * (r >> 2) + 4 * h2 + (r & 3)) * D + 32 * (j0 + j) + l32];
  }
  // stage the loaded piece and the state (S^T in bf16: row d_v, 4 consecutive d_k per write)
  auto stage = [&]() {
    kr.store(ks_);
    vr.store(vs_);
    qr.store(qs_);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *(bf16x4 *)(ss_ + tile_off<D>(32 * (j0 + j) + l32, 32 * iv + 8 * rq + 4 * h2)) =
            bf16x4{(__bf16)st[j][4 * rq], (__bf16)st[j][4 * rq + 1], (__bf16)st[j][4 * rq + 2], (__bf16)st[j][4 * rq + 3]};
  };
  load(row_begin);
  stage();
  __syncthreads();
  for (int c = 0; c < np; ++c) {
    const int r0 = row_begin + c * CR, nrows = min(CR, p.S - r0);
    const bool more = c + 1 < np;
    if (more) load(r0 + CR);
    f32x16 acc[DBW];
#pragma unroll
    for (int i = 0; i < DBW; ++i) acc[i] = f32x16{};
    // inside the piece: key blocks 0..qb (the wave's queries precede later keys)
    for (int kb = 0; kb <= qb; ++kb) {
      f32x16 s = f32x16{};
#pragma unroll 2
      for (int ks = 0; ks < KS; ++ks) s = mfma32(row_frag<D>(ks_, 32 * kb, ks, lane), row_frag<D>(qs_, 32 * qb, ks, lane), s);
      // s[r]: key 32 kb + 8(r/4) + 4h2 + r%4 of query row; mask keys past the query
      bf16x8 pk[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb + 8 * (r >> 2) + 4 * h2 + (r & 3);
        pk[r >> 3][r & 7] = (__bf16)(kb < qb || key <= row ? s[r] : 0.f);
      }
#pragma unroll
      for (int i = 0; i < DBW; ++i)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          acc[i] = mfma32(tr_frag<D>(vs_, 32 * kb + 16 * hh, 32 * (db0 + i), lane), pk[hh], acc[i]);
    }
    // earlier rows through the state before this piece: O^T += S^T . Q^T
#pragma unroll
    for (int i = 0; i < DBW; ++i)
#pragma unroll 2
      for (int ks = 0; ks < KS; ++ks)
        acc[i] = mfma32(row_frag<D>(ss_, 32 * (db0 + i), ks, lane), row_frag<D>(qs_, 32 * qb, ks, lane), acc[i]);
    if (more) {
      // the state after this piece, then the next piece into LDS
#pragma unroll
      for (int ks = 0; ks < CR / 16; ++ks) {
        const bf16x8 a = tr_frag<D>(ks_, 16 * ks, 32 * iv, lane);
#pragma unroll
        for (int j = 0; j < NJ; ++j) st[j] = mfma32(a, tr_frag<D>(vs_, 16 * ks, 32 * (j0 + j), lane), st[j]);
      }
      __syncthreads();
      stage();
      __syncthreads();
    }
    // the stores drain while the next piece is computed
    if (row < nrows) store_o<D, DBW>(p, acc, db0, b * p.o_sb + h * p.o_sh + (int64_t)(r0 + row) * p.o_ss, h2);
  }
}

// Sub-segment length and count for B * Hkv heads of S rows.
struct LinPlan {
  int64_t T, sub_len, n_sub;
};

LinPlan lin_plan(int64_t B, int64_t Hkv, int64_t S, int64_t D) {
  LinPlan pl;
  pl.T = (S + kChunk - 1) / kChunk;
  const int64_t want = std::max<int64_t>(1, kFill / std::max<int64_t>(1, B * Hkv));
  pl.sub_len = std::max<int64_t>(1, (pl.T + want - 1) / want);
  pl.n_sub = (pl.T + pl.sub_len - 1) / pl.sub_len;
  return pl;
}

template <int D>
hipError_t launch_d(LinAttnParams p, hipStream_t s) {
  const LinPlan pl = lin_plan(p.B, p.Hkv, p.S, D);
  p.sub_len = (int32_t)pl.sub_len;
  p.n_sub = (int32_t)pl.n_sub;
  p.seg_subs = std::max(1, std::min(p.Hq / p.Hkv, p.n_sub));
  p.n_seg = (p.n_sub + p.seg_subs - 1) / p.seg_subs;
  // the first pass reads only K and V: one workgroup per CU does best, each
  // taking consecutive sub-segments
  const int64_t heads = (int64_t)p.B * p.Hkv;
  p.sub_per_wg = (int32_t)std::max<int64_t>(1, heads * p.n_sub / kSubFill);
  const int64_t sub_wgs = heads * ((p.n_sub + p.sub_per_wg - 1) / p.sub_per_wg);
  if (p.n_sub > 0) hipLaunchKernelGGL(lin_sub_kernel<D>, dim3(sub_wgs), dim3(256), 0, s, p);
  if (p.n_seg > 0 || p.s_out)
    hipLaunchKernelGGL(lin_scan_kernel<D>, dim3(p.B * p.Hkv * (D * D / 1024)), dim3(256), 0, s, p);
  if (p.n_seg > 0) hipLaunchKernelGGL(lin_out_kernel<D>, dim3(p.B * p.Hq * p.n_seg), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// Workspace: [sub-segment sums, f32 | segment start states, f32], each
// [B, Hkv, n_sub, D_k, D_v].
void linear_attn_workspace_layout(int64_t B, int64_t Hkv, int64_t S, int64_t D, size_t off[3]) {
  const LinPlan pl = lin_plan(B, Hkv, S, D);
  const size_t per = (size_t)B * Hkv * pl.n_sub * D * D * 4;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  off[0] = 0;
  off[1] = up(per);
  off[2] = off[1] + up(per);
}

size_t linear_attn_workspace_bytes(int64_t B, int64_t Hkv, int64_t S, int64_t D) {
  size_t off[3];
  linear_attn_workspace_layout(B, Hkv, S, D, off);
  return off[2];
}

hipError_t launch_linear_attn(const LinAttnParams &p, int D, hipStream_t s) {
  // no rows and no state to pass: nothing to launch
  if (p.B == 0 || p.Hkv == 0 || (p.S == 0 && !p.s_out)) return hipSuccess;
  return D == 64 ? launch_d<64>(p, s) : launch_d<128>(p, s);
}

}  // namespace chain
