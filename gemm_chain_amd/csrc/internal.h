// Internal declarations shared by the host entry points and the gfx950 kernels.
//
// The schedule helpers here are __host__ __device__ so that the kernels and the
// host-side census / unit tests evaluate exactly the same tile classification
// and work-item mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "chain.h"

namespace chain {

constexpr int kMaxRanges = 2 * CHAIN_MAX_CHUNKS;  // key visit ranges
constexpr int kMaxRuns = CHAIN_MAX_RUNS;          // query position runs
constexpr int kNumXcd = 8;                        // MI355X: 8 XCDs, round-robin dispatch

// Key rows [beg[i], end[i]) of the K/V tensor are visited in order i = 0..n-1;
// a key row j of range i has global position j + pos_off[i].
struct KeyRanges {
  int32_t n;
  int32_t beg[kMaxRanges];
  int32_t end[kMaxRanges];
  int32_t pos_off[kMaxRanges];
};

// Query rows: run i starts at row row_beg[i]; a row of run i has position
// row + pos_off[i].  Positions strictly increase with the row.
struct RowRuns {
  int32_t n;
  int32_t row_beg[kMaxRuns];
  int32_t pos_off[kMaxRuns];
};

__host__ __device__ inline int32_t row_position(const RowRuns &r, int32_t row) {
  int32_t off = r.pos_off[0];
#pragma unroll
  for (int i = 1; i < kMaxRuns; ++i)
    if (i < r.n && row >= r.row_beg[i]) off = r.pos_off[i];
  return row + off;
}

enum TileClass : int { TILE_SKIP = 0, TILE_FULL = 1, TILE_DIAG = 2 };

// Query rows with positions in [qmin, qmax] against a key tile with positions
// [kmin, kmax]; `ragged` marks a key tile cut short by its range end.
// Written with selects only: on the GPU this runs once per tile in the loop.
__host__ __device__ inline int classify_tile(int causal, int32_t qmin, int32_t qmax,
                                             int32_t kmin, int32_t kmax, bool ragged) {
  const bool skip = (causal != 0) & (kmin > qmax);
  const bool diag = ragged | ((causal != 0) & (kmax > qmin));
  return skip ? TILE_SKIP : diag ? TILE_DIAG : TILE_FULL;
}

// Block ids are dealt to the XCDs round-robin (id % 8).  Map them so that XCD x
// receives the contiguous item range [x*q + min(x, r), ...): consecutive items
// (same batch and head group, neighbouring query tiles) then share one L2.
// A bijection of [0, n).
__host__ __device__ inline int32_t xcd_remap(int32_t bid, int32_t n) {
  const int32_t x = bid % kNumXcd, q = n / kNumXcd, r = n % kNumXcd;
  return x * q + (x < r ? x : r) + bid / kNumXcd;
}

// Fused-mode visit order over Sk keys: chunk s = contiguous range s of
// n_chunks, or (zigzag) the pieces s and 2*n_chunks-1-s of 2*n_chunks.
inline void build_fused_ranges(int64_t Sk, int n_chunks, int zigzag, KeyRanges *kr) {
  kr->n = 0;
  if (Sk == 0) return;
  if (!zigzag) {
    const int64_t n = Sk / n_chunks;
    for (int s = 0; s < n_chunks; ++s) {
      kr->beg[kr->n] = (int32_t)(s * n);
      kr->end[kr->n] = (int32_t)((s + 1) * n);
      kr->pos_off[kr->n++] = 0;
    }
  } else {
    const int64_t n = Sk / (2 * n_chunks);
    for (int s = 0; s < n_chunks; ++s) {
      const int64_t pieces[2] = {s, 2 * n_chunks - 1 - s};
      for (int k = 0; k < 2; ++k) {
        kr->beg[kr->n] = (int32_t)(pieces[k] * n);
        kr->end[kr->n] = (int32_t)((pieces[k] + 1) * n);
        kr->pos_off[kr->n++] = 0;
      }
    }
  }
}

// Ranges of a partial step: one per non-empty run of the key positions.
inline void build_run_ranges(const chain_segs &segs, KeyRanges *kr) {
  kr->n = 0;
  int64_t row = 0;
  for (int i = 0; i < segs.n; ++i) {
    if (segs.len[i] == 0) continue;
    kr->beg[kr->n] = (int32_t)row;
    kr->end[kr->n] = (int32_t)(row + segs.len[i]);
    kr->pos_off[kr->n++] = (int32_t)(segs.start[i] - row);
    row += segs.len[i];
  }
}

inline void build_row_runs(const chain_segs *segs, int64_t Sq, RowRuns *rr) {
  if (segs == nullptr) {
    rr->n = 1;
    rr->row_beg[0] = 0;
    rr->pos_off[0] = 0;
    return;
  }
  rr->n = 0;
  int64_t row = 0;
  for (int i = 0; i < segs->n; ++i) {
    if (segs->len[i] == 0) continue;
    rr->row_beg[rr->n] = (int32_t)row;
    rr->pos_off[rr->n++] = (int32_t)(segs->start[i] - row);
    row += segs->len[i];
  }
  if (rr->n == 0) {  // no rows at all
    rr->n = 1;
    rr->row_beg[0] = 0;
    rr->pos_off[0] = 0;
  }
  (void)Sq;
}

// Everything an attention kernel needs; passed by value as the kernel argument.
struct AttnParams {
  const void *q;
  const void *k;
  const void *v;
  void *o;
  float *lse;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t l_sb, l_sh, l_ss;
  int32_t B, Hq, Hkv, Sq, Sk;
  int32_t causal;
  int32_t o_f32;         // 1: O is f32, 0: O has the input dtype
  float scale_log2;      // scale * log2(e): scores are kept in base-2 units
  RowRuns qruns;
  KeyRanges kr;
};

struct MergeParams {
  const float *o_parts;
  const float *lse_parts;
  void *o;
  float *lse;
  int64_t p_sc, p_sb, p_sh, p_ss;   // O_parts strides
  int64_t lp_sc, lp_sb, lp_sh, lp_ss;  // LSE_parts strides
  int64_t o_sb, o_sh, o_ss;
  int64_t l_sb, l_sh, l_ss;
  int32_t C, B, H, S, D;
  int32_t o_f32;
};

struct GemmParams {
  const void *a;      // [M, K], row stride lda (k contiguous)
  const void *b;      // [K, N]: element (k, n) at b[k * b_sk + n * b_sn]; b_sk == 1 or b_sn == 1
  void *c;            // [M, N], row stride ldc (n contiguous)
  int64_t lda, b_sk, b_sn, ldc;
  int32_t M, N, K;
  int32_t act;        // chain_act
  int32_t c_f32;      // 1: C is f32, 0: C is bf16
  int32_t c_vec;      // 1: C rows allow 4-element vector stores (aligned base and ldc)
  const void *b2;     // gated: the up weights, strides of b; C = act(A.B) * (A.B2)
  int32_t gated;      // 1: the gated product above (bf16; b_sk == 1, or b_sn == 1 and gemm_gated_rowmajor_ok)
};

struct AttnBwdParams {
  const void *q, *k, *v, *o, *dout;   // bf16
  const float *lse;                   // natural log, [B, Hq, S]
  float *dq, *dk, *dv;                // outputs, f32
  float *rowv;                        // workspace: per (b, h), rows padded to a multiple of 64,
                                      // blocks of 16 rows [16 x -LSE*log2(e) | 16 x -D_i]
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t do_sb, do_sh, do_ss;
  int64_t l_sb, l_sh, l_ss;
  int64_t dq_sb, dq_sh, dq_ss;
  int64_t dk_sb, dk_sh, dk_ss;
  int64_t dv_sb, dv_sh, dv_ss;
  int32_t B, Hq, Hkv, S;
  int32_t causal;
  float scale;        // multiplies Q.K^T
  float scale_log2;   // scale * log2(e)
};

struct LinAttnParams {
  const void *q, *k, *v;              // bf16 [B, Hq|Hkv, S, D]
  void *o;                            // [B, Hq, S, D], f32 or bf16
  const float *s_in;                  // [B, Hkv, D_k, D_v] or null (zero state)
  float *s_out;                       // [B, Hkv, D_k, D_v] or null
  float *sub_total;                   // workspace: per sub-segment, the sum of its chunks' K^T V (f32, [D_k, D_v])
  float *seg_base;                    // workspace: per segment, the state at its start (f32, [D_k, D_v])
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t si_sb, si_sh, si_sr;
  int64_t so_sb, so_sh, so_sr;
  int32_t B, Hq, Hkv, S;
  int32_t o_f32;
  int32_t sub_len, n_sub;             // chunks per sub-segment; sub-segments per head
  int32_t seg_subs, n_seg;            // sub-segments per segment; segments per head
  int32_t sub_per_wg;                 // sub-segments per workgroup of the first pass
};

// Launchers (defined in the .hip files).  Each returns the launch's hipError_t.
hipError_t launch_attn_mfma_bf16(const AttnParams &p, int D, hipStream_t stream);
hipError_t launch_attn_valu(const AttnParams &p, int D, int dtype, hipStream_t stream);
hipError_t launch_lse_merge(const MergeParams &p, hipStream_t stream);
hipError_t launch_gemm(const GemmParams &p, int dtype, hipStream_t stream);
// Gated, with row-major gate and up weights (b_sn == 1): whether the kernel
// takes them (16-byte aligned bases, row stride and N multiples of 8, a tile's
// rows within 32-bit byte offsets).
bool gemm_gated_rowmajor_ok(const GemmParams &p);
hipError_t launch_attn_bwd(const AttnBwdParams &p, int D, hipStream_t stream);
hipError_t launch_linear_attn(const LinAttnParams &p, int D, hipStream_t stream);
size_t linear_attn_workspace_bytes(int64_t B, int64_t Hkv, int64_t S, int64_t D);
void linear_attn_workspace_layout(int64_t B, int64_t Hkv, int64_t S, int64_t D, size_t off[3]);

}  // namespace chain
