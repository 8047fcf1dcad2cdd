/*
 * libchain -- the two-matmul chain O = f(A.B).C on AMD Instinct MI355X (gfx950).
 *
 * The operation (METP article, FITEE doi 10.1631/FITEE.2400602, abstract): the
 * core unit of Transformer training is two consecutive matrix products with an
 * optional function between them.  Two instances are provided:
 *
 *   attention  A = Q, B = K^T, C = V, f = row softmax of scale * scores under an
 *              optional causal mask over global positions (TSP article, section
 *              "Lo que realmente significa plegar": causal attention needs the
 *              whole key/value context, which arrives reordered in zigzag
 *              pieces); query heads may share key/value heads in contiguous
 *              groups (2D-Attention summary, "Comprendiendo la Arquitectura de
 *              los LLMs": GQA).  Every row also yields its log-sum-exp
 *              LSE_i = log sum_j exp(s_ij), natural log, over visible keys j.
 *   MLP        A = X, B = W1, C = W2, f = GeLU (exact erf form, tanh form, or
 *              identity).
 *
 * Chunked evaluation and merging (2D-Attention summary, "Introduciendo la
 * Atencion 2D": tensors are chunked along the context; TSP article: partial
 * outputs are accumulated locally): attention over a union of disjoint key
 * sets equals the log-sum-exp merge of the per-set results,
 *   M = max_c LSE_c,  w_c = exp(LSE_c - M),  LSE = M + log sum w_c,
 *   O = sum_c w_c O_c / sum_c w_c,
 * with parts whose LSE is -inf ignored.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Memory: every tensor's data lives in device memory of the current HIP
 *   device; the caller allocates and owns all of it (including the MLP
 *   workspace).  The library never allocates or frees device memory and keeps
 *   no state between calls other than a thread-local error message, except
 *   chain_mlp_fwd_noalloc's static per-GPU scratch (described there).
 * - Layout: chain_tensor gives shape and strides in ELEMENTS; the last
 *   dimension must be contiguous (stride 1), other strides are free (>= 0);
 *   the MLP weights may instead have their first dimension contiguous.
 *   Attention tensors are [B, H, S, D]; LSE tensors are [B, H, S]; partial
 *   tensors carry a leading chunk dimension [C, B, H, S, D] / [C, B, H, S].
 * - Alignment (CHAIN_ERR_ALIGN otherwise): for tensors whose rows the kernels
 *   move as 16-byte vectors (Q, K, V, attention O, O_parts, X, W1, W2) the
 *   data pointer and every non-contiguous stride times the element size must
 *   be multiples of 16 bytes; 8 bytes for a bf16 merge output; LSE tensors and
 *   the MLP output only need element alignment (an MLP output whose pointer
 *   and row stride are multiples of 4 elements is written with vector stores).
 * - Streams: `stream` is a hipStream_t (NULL = the default stream).  Calls
 *   only enqueue work on it and return at once; results are visible after the
 *   caller synchronises the stream.  Calls are reentrant; concurrent calls on
 *   different streams are independent.
 * - Errors: arguments are validated synchronously before anything is
 *   launched; a call that fails validation has no side effect and returns a
 *   status other than CHAIN_OK, with details in chain_last_error().  A failed
 *   launch returns CHAIN_ERR_HIP.  Device faults surface at the caller's next
 *   synchronisation, as for any HIP work.
 * - Aliasing: outputs must not overlap inputs (CHAIN_ERR_ALIAS).
 * - Empty inputs: zero-sized batch, head or query dimensions are valid and
 *   launch nothing.
 */
#ifndef CHAIN_H
#define CHAIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CHAIN_VERSION 100           /* 1.0.0 */
#define CHAIN_MAX_DIMS 5
#define CHAIN_MAX_RUNS 4            /* position runs per chain_segs */
#define CHAIN_MAX_CHUNKS 64         /* n_chunks limit of chain_attn_fwd */

typedef enum {
  CHAIN_OK = 0,
  CHAIN_ERR_NULL = 1,         /* a required pointer is NULL */
  CHAIN_ERR_DTYPE = 2,        /* unsupported or mismatched element type */
  CHAIN_ERR_SHAPE = 3,        /* inconsistent shapes or chunk counts */
  CHAIN_ERR_LAYOUT = 4,       /* last dimension not contiguous, negative stride */
  CHAIN_ERR_ALIGN = 5,        /* pointer or stride not 16-byte aligned */
  CHAIN_ERR_ALIAS = 6,        /* an output overlaps an input */
  CHAIN_ERR_UNSUPPORTED = 7,  /* valid request outside what the kernels cover */
  CHAIN_ERR_WORKSPACE = 8,    /* MLP workspace missing or too small */
  CHAIN_ERR_HIP = 9           /* the HIP runtime reported an error */
} chain_status;

typedef enum { CHAIN_F32 = 0, CHAIN_BF16 = 1 } chain_dtype;

typedef enum {
  CHAIN_ACT_GELU_ERF = 0,     /* x * Phi(x) */
  CHAIN_ACT_GELU_TANH = 1,    /* x/2 * (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */
  CHAIN_ACT_IDENTITY = 2,
  CHAIN_ACT_SILU = 3          /* x / (1 + exp(-x)) */
} chain_act;

/* A strided view of device memory.  dtype is a chain_dtype. */
typedef struct {
  void *data;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[CHAIN_MAX_DIMS];
  int64_t stride[CHAIN_MAX_DIMS];
} chain_tensor;

/* Global sequence positions of the rows of a tensor, as n runs of consecutive
 * positions: row sum_{r'<r} len[r'] + t has position start[r] + t.  Runs must
 * be in ascending order and must not overlap (start[r+1] >= start[r]+len[r]),
 * so positions strictly increase with the row index.  Host memory. */
typedef struct {
  int32_t n;
  int64_t start[CHAIN_MAX_RUNS];
  int64_t len[CHAIN_MAX_RUNS];
} chain_segs;

/* Library version (CHAIN_VERSION of the build). */
int chain_version(void);

/* Static text naming a status. */
const char *chain_status_str(chain_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char *chain_last_error(void);

/*
 * chain_attn_fwd -- whole attention of Q against K/V, the key/value context
 * visited chunk by chunk with an online softmax (running max and log-sum-exp)
 * merge kept on chip, so O and LSE are final.
 *
 *   Q   [B, Hq, S, D]   f32 or bf16            (input)
 *   K,V [B, Hkv, S, D]  same dtype as Q        (input), Hq % Hkv == 0,
 *                       query head h uses key/value head h / (Hq / Hkv)
 *   O   [B, Hq, S, D]   same dtype as Q        (output)
 *   LSE [B, Hq, S]      f32, natural log       (output)
 *   causal   nonzero: key j visible to query i iff j <= i
 *   scale    multiplies Q.K^T (finite, usually 1/sqrt(D))
 *   n_chunks 1..CHAIN_MAX_CHUNKS key chunks visited in order 0..n_chunks-1;
 *            S must be a multiple of n_chunks (of 2*n_chunks with zigzag)
 *   zigzag   nonzero: chunk s is the pieces s and 2*n_chunks-1-s of a split
 *            of S into 2*n_chunks equal pieces (TSP article, zigzag partition);
 *            zero: chunk s is the s-th of n_chunks contiguous ranges
 * The result does not depend on n_chunks/zigzag beyond floating-point
 * rounding.  bf16 inputs: products are bf16 MFMAs with f32 accumulation; Q
 * times scale * log2(e) and the probabilities are rounded to bf16 as MFMA
 * operands; f32 inputs are computed in f32 throughout.  D must be 64 or 128,
 * and for bf16 the key (and the value) rows
 * of one head must span less than 2^31 bytes, i.e. ((S - 1) * stride + D) * 2
 * < 2^31 (CHAIN_ERR_UNSUPPORTED otherwise).
 */
chain_status chain_attn_fwd(const chain_tensor *Q, const chain_tensor *K,
                            const chain_tensor *V, const chain_tensor *O,
                            const chain_tensor *LSE, int causal, float scale,
                            int n_chunks, int zigzag, void *stream);

/*
 * chain_attn_partial -- one step of ring / zigzag sequence-parallel attention
 * (TSP article, "Lo que realmente significa plegar"; 2D-Attention summary,
 * "Introduciendo la Atencion 2D"): local queries attend to one arriving
 * key/value chunk and produce a partial result for chain_lse_merge.
 *
 *   Q        [B, Hq, Sq, D]   f32 or bf16, rows at positions q_pos   (input)
 *   Kc, Vc   [B, Hkv, Sk, D]  same dtype, rows at positions kv_pos   (input)
 *   O_part   [B, Hq, Sq, D]   f32                                    (output)
 *   LSE_part [B, Hq, Sq]      f32                                    (output)
 *   q_pos, kv_pos  host chain_segs covering exactly Sq and Sk rows
 * With causal, key j is visible to query i iff kv_pos(j) <= q_pos(i).  A row
 * that sees no key gets O_part = 0 and LSE_part = -inf (never NaN).
 * Sk == 0 is valid (every row is then such a row).  D must be 64 or 128; the
 * 2^31-byte limit on one head's key/value rows applies as for chain_attn_fwd.
 */
chain_status chain_attn_partial(const chain_tensor *Q, const chain_tensor *Kc,
                                const chain_tensor *Vc, const chain_tensor *O_part,
                                const chain_tensor *LSE_part, int causal, float scale,
                                const chain_segs *q_pos, const chain_segs *kv_pos,
                                void *stream);

/*
 * chain_lse_merge -- combine C partial results by log-sum-exp (formula above).
 *
 *   O_parts   [C, B, H, S, D]  f32   (input)
 *   LSE_parts [C, B, H, S]     f32   (input)
 *   O         [B, H, S, D]     f32 or bf16 (output, rounded to nearest even)
 *   LSE       [B, H, S]        f32   (output; may be NULL to skip it)
 * Rows whose parts are all -inf give O = 0, LSE = -inf.  1 <= C <= 64.
 * D must be a multiple of 4 and at most 256.  Sizes: S and B*H below 2^31 and
 * B*H*ceil(S/8) below 2^31, else CHAIN_ERR_UNSUPPORTED.
 */
chain_status chain_lse_merge(const chain_tensor *O_parts, const chain_tensor *LSE_parts,
                             const chain_tensor *O, const chain_tensor *LSE, void *stream);

/*
 * chain_mlp_fwd -- O = act(X.W1).W2 (METP article, abstract; TSP article: one
 * weight shard of the MLP ring).
 *
 *   X  [M, K]   bf16 or f32 (input, row-major)
 *   W1 [K, N]   same dtype (input)       W2 [N, K2]  same dtype (input)
 *               Each weight is row-major (stride (ld, 1)) or column-major
 *               (stride (1, ld)): the transpose of a row-major [N, K] array,
 *               the layout linear layers keep their weights in.  Column-major
 *               weights are the faster form (both operands stream along k).
 *   O  [M, K2]  bf16 or f32 (output, row-major)
 *   workspace   device buffer of at least chain_mlp_workspace_bytes(M, N, dtype)
 *               bytes, 256-byte aligned; holds H = act(X.W1) in the input dtype
 *               (bf16 H is rounded to nearest even, as the second product's
 *               MFMA operand).  Owned by the caller; contents are scratch.
 * Accumulation is f32.  K, N, K2 must be multiples of 8 and row strides at
 * most 2^25 elements (CHAIN_ERR_UNSUPPORTED otherwise).
 */
chain_status chain_mlp_fwd(const chain_tensor *X, const chain_tensor *W1,
                           const chain_tensor *W2, const chain_tensor *O, int act,
                           void *workspace, size_t ws_bytes, void *stream);

/* Bytes of workspace chain_mlp_fwd needs for an M x N intermediate of dtype
 * dt (a chain_dtype), rounded up to 256.  0 for an invalid dtype. */
size_t chain_mlp_workspace_bytes(int64_t M, int64_t N, int32_t dt);

/* Size of the static device scratch behind chain_mlp_fwd_noalloc: 64 MiB on
 * each GPU the library runs the call on, held until the process ends. */
#define CHAIN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * chain_mlp_fwd_noalloc -- chain_mlp_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, kernels and results as
 * chain_mlp_fwd, without the workspace: H = act(X.W1) lives in a static
 * device array of CHAIN_NOALLOC_SCRATCH_BYTES per GPU.
 *
 *   X, W1, W2, O, act, stream   as for chain_mlp_fwd
 * The call allocates nothing (no hipMalloc, no library allocation).  The
 * first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress, current device); a failure there returns
 * CHAIN_ERR_HIP.  Shapes whose H needs more than CHAIN_NOALLOC_SCRATCH_BYTES
 * (chain_mlp_workspace_bytes(M, N, dtype)) return CHAIN_ERR_WORKSPACE before
 * anything runs; for bf16 that is M * N <= 32 Mi elements.  Every call on a
 * GPU shares that GPU's array, which keeps the last call's H: calls that
 * overlap on one GPU (different streams, or threads without ordering) race
 * and give wrong results.  Calls ordered on one stream are safe.
 */
chain_status chain_mlp_fwd_noalloc(const chain_tensor *X, const chain_tensor *W1,
                                   const chain_tensor *W2, const chain_tensor *O, int act,
                                   void *stream);

/*
 * chain_mlp_gated_fwd -- O = (act(X.Wg) * (X.Wu)).Wd, * elementwise: the gated MLP
 * whose gate, up and down projection shards the TSP article circulates ("Lo que
 * realmente significa plegar"); the activation acts on the gate product only.
 *
 *   X      [M, K]    bf16 (input, row-major)
 *   Wg, Wu [K, N]    bf16 (input), both column-major (stride (1, ld)): the
 *                    transpose of row-major [N, K] weights, as linear layers store
 *                    them; or both row-major (stride (ld, 1)); the two with the
 *                    same strides
 *   Wd     [N, K2]   bf16 (input), row- or column-major as W2 of chain_mlp_fwd
 *   O      [M, K2]   bf16 or f32 (output, row-major)
 *   act    a chain_act (CHAIN_ACT_SILU is the usual gate)
 *   workspace  as for chain_mlp_fwd: chain_mlp_workspace_bytes(M, N, CHAIN_BF16)
 *              bytes, 256-byte aligned, holding H = act(X.Wg) * (X.Wu) in bf16
 *              (rounded to nearest even after the f32 product).
 * One kernel computes both products of a tile and the gate in its epilogue;
 * accumulation is f32; both weight layouts give the same bits.  K, N, K2
 * multiples of 8; f32 inputs, gate and up weights of different layouts or
 * strides, or row-major ones whose K rows span 2^31 bytes or more give
 * CHAIN_ERR_UNSUPPORTED.  Other conventions as chain_mlp_fwd.
 */
chain_status chain_mlp_gated_fwd(const chain_tensor *X, const chain_tensor *Wg,
                                 const chain_tensor *Wu, const chain_tensor *Wd,
                                 const chain_tensor *O, int act, void *workspace,
                                 size_t ws_bytes, void *stream);

/*
 * chain_attn_bwd -- gradients of chain_attn_fwd's attention (bf16, whole key
 * context, positions 0..S-1) with respect to Q, K and V.  The pages treat the
 * chain as the core unit of Transformer training (METP article, abstract) and
 * keep only what the backward needs, recomputing the rest (2D-Attention
 * summary, "Estrategias de Entrenamiento Distribuido"); the gradient itself is
 * the chain rule of the forward definition: with P_ij = exp(scale*s_ij - LSE_i)
 * on visible keys, D_i = sum_d dO_id O_id and dS = P * (dO.V^T - D),
 *   dQ = scale * dS.K,   dK = scale * dS^T.Q,   dV = P^T.dO,
 * dK and dV summed over the query heads that share a key/value head.
 *
 *   Q    [B, Hq, S, D]   bf16   (input)
 *   K, V [B, Hkv, S, D]  bf16   (input), Hq % Hkv == 0, grouping as in chain_attn_fwd
 *   O    [B, Hq, S, D]   bf16   (input: chain_attn_fwd's output)
 *   LSE  [B, Hq, S]      f32    (input: chain_attn_fwd's log-sum-exp, natural log)
 *   dO   [B, Hq, S, D]   bf16   (input: gradient of the loss with respect to O)
 *   dQ   [B, Hq, S, D]   f32    (output)
 *   dK,dV [B, Hkv, S, D] f32    (output)
 *   causal, scale  as given to chain_attn_fwd
 *   workspace  device buffer of at least chain_attn_bwd_workspace_bytes(B, Hq, S)
 *              bytes, 256-byte aligned; caller-owned scratch (holds -D_i and
 *              -LSE_i * log2(e) per row)
 * P is recomputed from Q, K and LSE, so LSE must be the one the forward
 * produced for these Q and K.  D must be 64 or 128.  Products are bf16 MFMAs
 * with f32 accumulation; the scores are formed from bf16 operands pre-scaled
 * by scale * log2(e) (Q in the dQ kernel, as in the forward; K in the dK/dV
 * kernel), and P and dS are rounded to bf16 as MFMA operands.
 * Every output element is written exactly once (no atomics), so repeated
 * calls give identical bits.  dQ, dK, dV and the workspace must not overlap
 * each other or any input (CHAIN_ERR_ALIAS).  Alignment: 16 bytes for all
 * tensors except LSE (4).  B * Hq * S must be below 2^31 (UNSUPPORTED).
 */
chain_status chain_attn_bwd(const chain_tensor *Q, const chain_tensor *K, const chain_tensor *V,
                            const chain_tensor *O, const chain_tensor *LSE, const chain_tensor *dO,
                            const chain_tensor *dQ, const chain_tensor *dK, const chain_tensor *dV,
                            int causal, float scale, void *workspace, size_t ws_bytes,
                            void *stream);

/* Bytes of workspace chain_attn_bwd needs, rounded up to 256; 0 for negative
 * sizes. */
size_t chain_attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t S);

/*
 * chain_linear_attn_fwd -- causal linear attention with a carried key/value state:
 * one device's share of linear-attention sequence parallelism (LASP summary,
 * abstract: an intermediate key/value state is handed from device to device;
 * right-product evaluation; the intermediate states are cached).  With no
 * normalisation and no decay (the page prints no formula), for query head h and
 * key/value head g = h / (Hq / Hkv):
 *   O_i   = sum_{j<=i} (q_i . k_j) v_j + q_i S_in,
 *   S_out = S_in + sum_j k_j^T v_j          (D x D, row d_k, column d_v)
 *
 *   Q      [B, Hq, S, D]    bf16 (input)
 *   K, V   [B, Hkv, S, D]   bf16 (input), Hq % Hkv == 0
 *   O      [B, Hq, S, D]    f32 or bf16 (output)
 *   S_in   [B, Hkv, D, D]   f32 (input; NULL = zero state, the first share)
 *   S_out  [B, Hkv, D, D]   f32 (output; NULL to skip)
 *   workspace  at least chain_linear_attn_workspace_bytes(B, Hkv, S, D) bytes,
 *              256-byte aligned; caller-owned scratch (the cached states, f32:
 *              per run of consecutive 128-row chunks the sum of their K^T V,
 *              and the state at the start of each run of such runs)
 * Products are bf16 MFMAs with f32 accumulation; the scores inside a piece of
 * rows (64 rows at D = 128, 128 at D = 64) and the f32 state before each piece
 * are rounded to bf16 as MFMA operands.  D must be 64 or 128.  The last
 * dimension of every tensor is contiguous; Q, K, V, O 16-byte aligned, the
 * states 4-byte aligned.
 * S == 0 is valid (S_out = S_in).  Outputs and workspace must not overlap inputs
 * or each other.
 */
chain_status chain_linear_attn_fwd(const chain_tensor *Q, const chain_tensor *K,
                                   const chain_tensor *V, const chain_tensor *O,
                                   const chain_tensor *S_in, const chain_tensor *S_out,
                                   void *workspace, size_t ws_bytes, void *stream);

/* Bytes of workspace chain_linear_attn_fwd needs (0 for negative sizes). */
size_t chain_linear_attn_workspace_bytes(int64_t B, int64_t Hkv, int64_t S, int64_t D);

/*
 * chain_zigzag_segs -- host helper: the positions of share r of `parts` in a
 * zigzag split of S tokens (TSP article, zigzag partition): the pieces r and
 * 2*parts-1-r of 2*parts equal pieces, as two runs in ascending order.  Used
 * both for a rank's query share and for zigzag key/value chunks.
 * S must be a positive multiple of 2*parts and 0 <= r < parts.
 */
chain_status chain_zigzag_segs(int64_t S, int32_t parts, int32_t r, chain_segs *out);

/*
 * chain_attn_tile_census -- host helper describing the causal tile schedule
 * that chain_attn_fwd / chain_attn_partial apply: over query tiles of
 * block_m rows and key tiles of block_n rows (tiles cut inside each run /
 * chunk range as the kernels cut them), count tiles fully visible (`full`),
 * partly visible (`diag`, masked element by element) and invisible (`skip`,
 * never computed).  kv_pos NULL means positions 0..Sk-1; n_chunks/zigzag as
 * in chain_attn_fwd (ignored when kv_pos is given).  Host only.
 */
chain_status chain_attn_tile_census(int64_t Sq, const chain_segs *q_pos, int64_t Sk,
                                    const chain_segs *kv_pos, int n_chunks, int zigzag,
                                    int causal, int block_m, int block_n,
                                    int64_t *full, int64_t *diag, int64_t *skip);

#ifdef __cplusplus
}
#endif

#endif /* CHAIN_H */
