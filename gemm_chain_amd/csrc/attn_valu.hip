// Attention on the vector ALUs in f32: the exact-precision path.
//
// Same definition as the MFMA kernel (METP abstract: the chain O = f(Q.K^T).V
// with f the scaled, masked row softmax; TSP article: causal over global
// positions; 2D-Attention summary: GQA head sharing), evaluated with f32
// products and sums, so f32 inputs keep f32 accuracy.  Each lane owns one query
// row; key/value tiles of 64 rows are staged in LDS as f32 and read by all
// lanes at the same address (broadcast, no bank conflicts).  Keys are visited
// in the caller's range order with an online softmax in base 2.
#include "internal.h"

namespace chain {
namespace {

constexpr int kTile = 64;

template <typename T>
__device__ inline float ld(const T *p) { return (float)*p; }

template <typename T, int D>
__global__ __launch_bounds__(64) void attn_valu_kernel(const AttnParams p) {
  __shared__ float ks[kTile][D];
  __shared__ float vs[kTile][D];
  const int b = blockIdx.z, h = blockIdx.y;
  const int g = h / (p.Hq / p.Hkv);
  const int row0 = blockIdx.x * 64;
  const int row = row0 + threadIdx.x;
  const bool valid = row < p.Sq;
  const int last = min(row0 + 63, p.Sq - 1);
  const int32_t qpos = row_position(p.qruns, valid ? row : last);
  const int32_t blk_qmax = row_position(p.qruns, last);

  float q[D], acc[D];
  const T *qrow = (const T *)p.q + b * p.q_sb + h * p.q_sh + (int64_t)(valid ? row : last) * p.q_ss;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = ld(qrow + d) * p.scale_log2;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const T *kb = (const T *)p.k + b * p.k_sb + g * p.k_sh;
  const T *vb = (const T *)p.v + b * p.v_sb + g * p.v_sh;
  for (int ri = 0; ri < p.kr.n; ++ri) {
    const int beg = p.kr.beg[ri], end = p.kr.end[ri], off = p.kr.pos_off[ri];
    for (int k0 = beg; k0 < end; k0 += kTile) {
      if (p.causal && k0 + off > blk_qmax) break;
      const int cnt = min(kTile, end - k0);
      __syncthreads();
      for (int i = threadIdx.x; i < kTile * D; i += 64) {
        const int r = i / D, c = i % D;
        float kv = 0.f, vv = 0.f;
        if (r < cnt) {
          kv = ld(kb + (int64_t)(k0 + r) * p.k_ss + c);
          vv = ld(vb + (int64_t)(k0 + r) * p.v_ss + c);
        }
        ks[r][c] = kv;
        vs[r][c] = vv;
      }
      __syncthreads();
      for (int j0 = 0; j0 < cnt; j0 += 16) {
        float s[16];
        float mx = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int j = j0 + jj;
          float acc_s = 0.f;
#pragma unroll
          for (int d = 0; d < D; ++d) acc_s = fmaf(q[d], ks[j][d], acc_s);
          const bool vis = j < cnt && (!p.causal || k0 + j + off <= qpos);
          s[jj] = vis ? acc_s : -INFINITY;
          mx = fmaxf(mx, s[jj]);
        }
        const float m_new = fmaxf(m, mx);
        if (m_new == -INFINITY) continue;  // nothing visible yet
        const float alpha = exp2f(m - m_new);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const float e = exp2f(s[jj] - m_new);
          l += e;
          const int j = min(j0 + jj, kTile - 1);
#pragma unroll
          for (int d = 0; d < D; ++d) acc[d] = fmaf(e, vs[j][d], acc[d]);
        }
        m = m_new;
      }
    }
  }
  if (!valid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t orow = b * p.o_sb + h * p.o_sh + (int64_t)row * p.o_ss;
  if (p.o_f32) {
    float *o = (float *)p.o + orow;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = acc[d] * inv;
  } else {
    T *o = (T *)p.o + orow;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = (T)(acc[d] * inv);
  }
  p.lse[b * p.l_sb + h * p.l_sh + (int64_t)row * p.l_ss] =
      l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

template <typename T, int D>
hipError_t launch(const AttnParams &p, hipStream_t s) {
  dim3 grid((p.Sq + 63) / 64, p.Hq, p.B);
  hipLaunchKernelGGL((attn_valu_kernel<T, D>), grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_valu(const AttnParams &p, int D, int dtype, hipStream_t s) {
  if (dtype == CHAIN_F32) return D == 64 ? launch<float, 64>(p, s) : launch<float, 128>(p, s);
  return D == 64 ? launch<__bf16, 64>(p, s) : launch<__bf16, 128>(p, s);
}

}  // namespace chain
