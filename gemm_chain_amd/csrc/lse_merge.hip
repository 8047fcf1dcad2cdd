// Log-sum-exp merge of partial attention results (HBM-bound streaming kernel).
//
// TSP article, "Lo que realmente significa plegar": each device accumulates the
// partial outputs it computes as pieces of the context arrive.  For C parts
// (O_c, LSE_c) over disjoint key sets: M = max_c LSE_c, w_c = exp(LSE_c - M),
// LSE = M + log sum w_c, O = sum_c w_c O_c / sum w_c; parts with LSE = -inf
// carry no weight, and all--inf rows give O = 0, LSE = -inf.
//
// 32 lanes per output row, each lane streaming 16-byte float4 slices of every
// part (coalesced 512-byte row segments per half-wave) with non-temporal
// loads: the partials are read exactly once.  The outputs go out as
// non-temporal stores too (about 7 % faster than plain stores, which share the
// cache with the partials' stream).  For the common part counts the
// count is a template parameter, so all C slices of a lane are requested before
// the first one is consumed (C x 16 bytes in flight per lane).  The C LSE values of a row are read by all
// 32 lanes at one address (one broadcast transaction).
#include "internal.h"

namespace chain {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerPass = 8;   // 256 threads = 8 rows of 32 lanes

struct RowRef {
  int b, h, s;
};

__device__ inline void store_row(const MergeParams &p, const RowRef &r, int j, f32x4 o) {
  const int64_t orow = r.b * p.o_sb + r.h * p.o_sh + (int64_t)r.s * p.o_ss;
  if (p.o_f32) {
    __builtin_nontemporal_store(o, (f32x4 *)((float *)p.o + orow + 4 * j));
  } else {
    bf16x4 w = {(__bf16)o.x, (__bf16)o.y, (__bf16)o.z, (__bf16)o.w};
    __builtin_nontemporal_store(w, (bf16x4 *)((__bf16 *)p.o + orow + 4 * j));
  }
}

__device__ inline void store_lse(const MergeParams &p, const RowRef &r, float v) {
  if (p.lse) __builtin_nontemporal_store(v, p.lse + r.b * p.l_sb + r.h * p.l_sh + (int64_t)r.s * p.l_ss);
}

// C known at compile time: all loads of a lane are issued before the first is
// consumed.  A workgroup covers RPB consecutive rows of one (batch, head): the
// (b, h) pair and the row block come from the workgroup index by two uniform
// 32-bit divisions, so no lane divides (64-bit row arithmetic per lane cost the
// kernel about a tenth of its time).  R rows per lane group: 2 for few parts,
// so that a lane still has 2 C x 16 bytes in flight; 1 for 8 and more parts,
// in 512-thread workgroups, which measured a little faster than 2 rows in 256.
template <int C, int R, int BS>
__global__ __launch_bounds__(BS) void lse_merge_fixed(const MergeParams p, const uint32_t nsb) {
  constexpr int RPB = BS / 32 * R;  // rows per workgroup
  const int lr = threadIdx.x & 31;
  const uint32_t bh = blockIdx.x / nsb;
  const int s0 = (int)(blockIdx.x - bh * nsb) * RPB + (int)(threadIdx.x >> 5) * R;
  const int b = (int)(bh / (uint32_t)p.H), h = (int)bh - b * p.H;
  const int nslices = p.D / 4;
  const float *lbase = p.lse_parts + b * p.lp_sb + h * p.lp_sh;
  const float *obase = p.o_parts + b * p.p_sb + h * p.p_sh;
  RowRef ref[R];
  bool live[R];
  float lse[R][C];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    live[i] = s0 + i < p.S;
    ref[i] = {b, h, live[i] ? s0 + i : 0};
    const float *lp = lbase + (int64_t)ref[i].s * p.lp_ss;
#pragma unroll
    for (int c = 0; c < C; ++c) lse[i][c] = lp[c * p.lp_sc];
  }
  for (int j = lr; j < nslices; j += 32) {
    f32x4 x[R][C];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float *op = obase + (int64_t)ref[i].s * p.p_ss + 4 * j;
#pragma unroll
      for (int c = 0; c < C; ++c) x[i][c] = __builtin_nontemporal_load((const f32x4 *)(op + c * p.p_sc));
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float M = -INFINITY;
#pragma unroll
      for (int c = 0; c < C; ++c) M = fmaxf(M, lse[i][c]);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      float wsum = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const float w = expf(lse[i][c] - M);   // exp(-inf) = 0 for empty parts
          wsum += w;
          acc += w * x[i][c];
        }
        acc *= 1.f / wsum;
      }
      if (live[i]) {
        store_row(p, ref[i], j, acc);
        if (j == lr && lr == 0) store_lse(p, ref[i], M == -INFINITY ? -INFINITY : M + logf(wsum));
      }
    }
  }
}

// Any C (up to 64): one row per lane group, parts streamed in order; the
// same per-workgroup (batch, head, row block) decomposition.
__global__ __launch_bounds__(256) void lse_merge_any(const MergeParams p, const uint32_t nsb) {
  const int lr = threadIdx.x & 31;
  const uint32_t bh = blockIdx.x / nsb;
  const int s = (int)(blockIdx.x - bh * nsb) * kRowsPerPass + (int)(threadIdx.x >> 5);
  if (s >= p.S) return;
  const int b = (int)(bh / (uint32_t)p.H), h = (int)bh - b * p.H;
  const RowRef r = {b, h, s};
  const float *lp = p.lse_parts + b * p.lp_sb + h * p.lp_sh + (int64_t)s * p.lp_ss;
  const float *op = p.o_parts + b * p.p_sb + h * p.p_sh + (int64_t)s * p.p_ss;
  float M = -INFINITY;
  for (int c = 0; c < p.C; ++c) M = fmaxf(M, lp[c * p.lp_sc]);
  const int nslices = p.D / 4;
  float wsum = 0.f;
  if (M != -INFINITY)
    for (int c = 0; c < p.C; ++c) wsum += expf(lp[c * p.lp_sc] - M);
  for (int j = lr; j < nslices; j += 32) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll 8
      for (int c = 0; c < p.C; ++c) {
        const float w = expf(lp[c * p.lp_sc] - M);
        acc += w * __builtin_nontemporal_load((const f32x4 *)(op + c * p.p_sc + 4 * j));
      }
      acc *= 1.f / wsum;
    }
    store_row(p, r, j, acc);
  }
  if (lr == 0) store_lse(p, r, M == -INFINITY ? -INFINITY : M + logf(wsum));
}

template <int C, int R, int BS>
hipError_t launch_fixed(const MergeParams &p, hipStream_t stream) {
  constexpr int RPB = BS / 32 * R;
  const int64_t nsb = ((int64_t)p.S + RPB - 1) / RPB;
  const int64_t blocks = nsb * p.B * p.H;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((lse_merge_fixed<C, R, BS>), dim3((unsigned)blocks), dim3(BS), 0, stream, p, (uint32_t)nsb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const MergeParams &p, hipStream_t stream) {
  switch (p.C) {
    case 1: return launch_fixed<1, 2, 256>(p, stream);
    case 2: return launch_fixed<2, 2, 256>(p, stream);
    case 4: return launch_fixed<4, 2, 256>(p, stream);
    case 8: return launch_fixed<8, 1, 512>(p, stream);
    case 16: return launch_fixed<16, 1, 512>(p, stream);
    default: break;
  }
  const int64_t nsb = ((int64_t)p.S + kRowsPerPass - 1) / kRowsPerPass;
  const int64_t blocks = nsb * p.B * p.H;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(lse_merge_any, dim3((unsigned)blocks), dim3(256), 0, stream, p, (uint32_t)nsb);
  return hipGetLastError();
}

}  // namespace chain
