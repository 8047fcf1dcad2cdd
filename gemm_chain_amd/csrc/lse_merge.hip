// Log-sum-exp merge of partial attention results (HBM-bound streaming kernel).
//
// TSP article, "Lo que realmente significa plegar": each device accumulates the
// partial outputs it computes as pieces of the context arrive.  For C parts
// (O_c, LSE_c) over disjoint key sets: M = max_c LSE_c, w_c = exp(LSE_c - M),
// LSE = M + log sum w_c, O = sum_c w_c O_c / sum w_c; parts with LSE = -inf
// carry no weight, and all--inf rows give O = 0, LSE = -inf.
//
// 32 lanes per output row, each lane streaming 16-byte float4 slices of every
// part (coalesced 512-byte row segments per half-wave).  The C LSE values of a
// row are read by all 32 lanes at one address (a single broadcast transaction).
#include "internal.h"

namespace chain {
namespace {

constexpr int kRowsPerBlock = 8;  // 256 threads = 8 rows of 32 lanes

__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeParams p) {
  const int lr = threadIdx.x & 31;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 5);
  const int64_t rows = (int64_t)p.B * p.H * p.S;
  if (row >= rows) return;
  const int s = (int)(row % p.S);
  const int h = (int)((row / p.S) % p.H);
  const int b = (int)(row / ((int64_t)p.S * p.H));
  const float *lp = p.lse_parts + b * p.lp_sb + h * p.lp_sh + (int64_t)s * p.lp_ss;
  const float *op = p.o_parts + b * p.p_sb + h * p.p_sh + (int64_t)s * p.p_ss;

  float M = -INFINITY;
  for (int c = 0; c < p.C; ++c) M = fmaxf(M, lp[c * p.lp_sc]);
  const int64_t orow = b * p.o_sb + h * p.o_sh + (int64_t)s * p.o_ss;
  const int nslices = p.D / 4;
  if (M == -INFINITY) {
    for (int j = lr; j < nslices; j += 32) {
      if (p.o_f32) *(float4 *)((float *)p.o + orow + 4 * j) = make_float4(0.f, 0.f, 0.f, 0.f);
      else *(uint2 *)((__bf16 *)p.o + orow + 4 * j) = make_uint2(0u, 0u);
    }
    if (p.lse && lr == 0) p.lse[b * p.l_sb + h * p.l_sh + (int64_t)s * p.l_ss] = -INFINITY;
    return;
  }
  float wsum = 0.f;
  float4 acc[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
#pragma unroll 8
  for (int c = 0; c < p.C; ++c) {
    const float w = expf(lp[c * p.lp_sc] - M);   // exp(-inf) = 0 for empty parts
    wsum += w;
    const float *src = op + c * p.p_sc;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = lr + 32 * jj;
      if (j < nslices) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 x = __builtin_nontemporal_load((const f32x4 *)(src + 4 * j));
        acc[jj].x = fmaf(w, x.x, acc[jj].x);
        acc[jj].y = fmaf(w, x.y, acc[jj].y);
        acc[jj].z = fmaf(w, x.z, acc[jj].z);
        acc[jj].w = fmaf(w, x.w, acc[jj].w);
      }
    }
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int j = lr + 32 * jj;
    if (j < nslices) {
      const float4 o = make_float4(acc[jj].x * inv, acc[jj].y * inv, acc[jj].z * inv, acc[jj].w * inv);
      if (p.o_f32) {
        *(float4 *)((float *)p.o + orow + 4 * j) = o;
      } else {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 w = {(__bf16)o.x, (__bf16)o.y, (__bf16)o.z, (__bf16)o.w};
        *(bf16x4 *)((__bf16 *)p.o + orow + 4 * j) = w;
      }
    }
  }
  if (p.lse && lr == 0) p.lse[b * p.l_sb + h * p.l_sh + (int64_t)s * p.l_ss] = M + logf(wsum);
}

}  // namespace

hipError_t launch_lse_merge(const MergeParams &p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.H * p.S;
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace chain
