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
// loads: the partials are read exactly once.  For the common part counts the
// count is a template parameter, so all C slices of a lane are requested before
// the first one is consumed (C x 16 bytes in flight per lane) and each lane
// works on two rows to double that.  The C LSE values of a row are read by all
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

__device__ inline RowRef row_ref(const MergeParams &p, int64_t row) {
  RowRef r;
  r.s = (int)(row % p.S);
  r.h = (int)((row / p.S) % p.H);
  r.b = (int)(row / ((int64_t)p.S * p.H));
  return r;
}

__device__ inline void store_row(const MergeParams &p, const RowRef &r, int j, f32x4 o) {
  const int64_t orow = r.b * p.o_sb + r.h * p.o_sh + (int64_t)r.s * p.o_ss;
  if (p.o_f32) {
    *(f32x4 *)((float *)p.o + orow + 4 * j) = o;
  } else {
    bf16x4 w = {(__bf16)o.x, (__bf16)o.y, (__bf16)o.z, (__bf16)o.w};
    *(bf16x4 *)((__bf16 *)p.o + orow + 4 * j) = w;
  }
}

__device__ inline void store_lse(const MergeParams &p, const RowRef &r, float v) {
  if (p.lse) p.lse[r.b * p.l_sb + r.h * p.l_sh + (int64_t)r.s * p.l_ss] = v;
}

// C known at compile time: two rows per lane group, all loads issued first.
template <int C>
__global__ __launch_bounds__(256) void lse_merge_fixed(const MergeParams p) {
  constexpr int R = 2;  // rows per lane group
  const int lr = threadIdx.x & 31;
  const int64_t rows = (int64_t)p.B * p.H * p.S;
  const int64_t row0 = ((int64_t)blockIdx.x * kRowsPerPass + (threadIdx.x >> 5)) * R;
  const int nslices = p.D / 4;
  RowRef ref[R];
  bool live[R];
  float lse[R][C];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    live[i] = row0 + i < rows;
    ref[i] = row_ref(p, live[i] ? row0 + i : 0);
    const float *lp = p.lse_parts + ref[i].b * p.lp_sb + ref[i].h * p.lp_sh + (int64_t)ref[i].s * p.lp_ss;
#pragma unroll
    for (int c = 0; c < C; ++c) lse[i][c] = lp[c * p.lp_sc];
  }
  for (int j = lr; j < nslices; j += 32) {
    f32x4 x[R][C];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float *op = p.o_parts + ref[i].b * p.p_sb + ref[i].h * p.p_sh + (int64_t)ref[i].s * p.p_ss + 4 * j;
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

// Any C (up to 64): one row per lane group, parts streamed in order.
__global__ __launch_bounds__(256) void lse_merge_any(const MergeParams p) {
  const int lr = threadIdx.x & 31;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerPass + (threadIdx.x >> 5);
  const int64_t rows = (int64_t)p.B * p.H * p.S;
  if (row >= rows) return;
  const RowRef r = row_ref(p, row);
  const float *lp = p.lse_parts + r.b * p.lp_sb + r.h * p.lp_sh + (int64_t)r.s * p.lp_ss;
  const float *op = p.o_parts + r.b * p.p_sb + r.h * p.p_sh + (int64_t)r.s * p.p_ss;
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

template <int C>
hipError_t launch_fixed(const MergeParams &p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.H * p.S;
  const int64_t blocks = (rows + 2 * kRowsPerPass - 1) / (2 * kRowsPerPass);
  hipLaunchKernelGGL(lse_merge_fixed<C>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const MergeParams &p, hipStream_t stream) {
  switch (p.C) {
    case 1: return launch_fixed<1>(p, stream);
    case 2: return launch_fixed<2>(p, stream);
    case 4: return launch_fixed<4>(p, stream);
    case 8: return launch_fixed<8>(p, stream);
    case 16: return launch_fixed<16>(p, stream);
    default: break;
  }
  const int64_t rows = (int64_t)p.B * p.H * p.S;
  const int64_t blocks = (rows + kRowsPerPass - 1) / kRowsPerPass;
  hipLaunchKernelGGL(lse_merge_any, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace chain
