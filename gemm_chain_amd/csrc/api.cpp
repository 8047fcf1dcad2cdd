// Host side of libchain: argument validation, schedule tables, dispatch.
//
// Every entry point validates all of its arguments before it launches
// anything, so a failed call has no side effect.  Launches go to the caller's
// stream; nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

chain_status fail(chain_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

chain_status ok() {
  g_last_error.clear();
  return CHAIN_OK;
}

size_t elem_size(int32_t dt) { return dt == CHAIN_F32 ? 4 : dt == CHAIN_BF16 ? 2 : 0; }

// Byte extent [lo, hi) covered by a tensor (empty tensors cover nothing).
struct Extent {
  uintptr_t lo = 0, hi = 0;
};

Extent extent(const chain_tensor &t) {
  Extent e;
  int64_t last = 0;
  for (int i = 0; i < t.ndim; ++i) {
    if (t.shape[i] == 0) return e;
    last += (t.shape[i] - 1) * t.stride[i];
  }
  e.lo = (uintptr_t)t.data;
  e.hi = e.lo + (uintptr_t)((last + 1) * (int64_t)elem_size(t.dtype));
  return e;
}

bool overlap(const chain_tensor &a, const chain_tensor &b) {
  const Extent x = extent(a), y = extent(b);
  if (x.lo == x.hi || y.lo == y.hi) return false;
  return x.lo < y.hi && y.lo < x.hi;
}

int64_t numel(const chain_tensor &t) {
  int64_t n = 1;
  for (int i = 0; i < t.ndim; ++i) n *= t.shape[i];
  return n;
}

// Structural checks common to every tensor argument.  `align` is the byte
// alignment the kernels need for the data pointer and every outer stride
// (16 where rows are moved as 16-byte vectors, the element size where a
// tensor is accessed element by element).
chain_status check_tensor(const chain_tensor *t, const char *name, int ndim, int align = 16,
                          bool either_major = false) {
  if (t == nullptr) return fail(CHAIN_ERR_NULL, "%s: descriptor is NULL", name);
  if (t->ndim != ndim) return fail(CHAIN_ERR_SHAPE, "%s: expected %d dims, got %d", name, ndim, t->ndim);
  if (elem_size(t->dtype) == 0) return fail(CHAIN_ERR_DTYPE, "%s: unknown dtype %d", name, t->dtype);
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0) return fail(CHAIN_ERR_SHAPE, "%s: negative shape[%d]", name, i);
    if (t->stride[i] < 0) return fail(CHAIN_ERR_LAYOUT, "%s: negative stride[%d]", name, i);
  }
  if (numel(*t) == 0) return CHAIN_OK;
  if (t->data == nullptr) return fail(CHAIN_ERR_NULL, "%s: data is NULL", name);
  // The contiguous dimension: the last one, or (either_major, 2-D) the first.
  int cdim = ndim - 1;
  if (either_major && ndim == 2 && !(t->shape[1] <= 1 || t->stride[1] == 1) &&
      (t->shape[0] <= 1 || t->stride[0] == 1))
    cdim = 0;
  if (t->shape[cdim] > 1 && t->stride[cdim] != 1)
    return fail(CHAIN_ERR_LAYOUT, either_major ? "%s: neither dimension is contiguous"
                                               : "%s: last dimension must be contiguous (stride %lld)",
                name, (long long)t->stride[cdim]);
  const size_t es = elem_size(t->dtype);
  if (((uintptr_t)t->data) % align)
    return fail(CHAIN_ERR_ALIGN, "%s: data pointer not %d-byte aligned", name, align);
  for (int i = 0; i < ndim; ++i)
    if (i != cdim && t->shape[i] > 1 && (t->stride[i] * (int64_t)es) % align)
      return fail(CHAIN_ERR_ALIGN, "%s: stride[%d] * %zu bytes not a multiple of %d", name, i, es, align);
  return CHAIN_OK;
}

chain_status check_segs(const chain_segs *s, int64_t rows, const char *name) {
  if (s == nullptr) return fail(CHAIN_ERR_NULL, "%s: NULL", name);
  if (s->n < 1 || s->n > CHAIN_MAX_RUNS)
    return fail(CHAIN_ERR_SHAPE, "%s: run count %d outside 1..%d", name, s->n, CHAIN_MAX_RUNS);
  int64_t total = 0, next_free = INT64_MIN;
  for (int i = 0; i < s->n; ++i) {
    if (s->len[i] < 0 || s->start[i] < 0)
      return fail(CHAIN_ERR_SHAPE, "%s: run %d has negative start or length", name, i);
    if (s->len[i] == 0) continue;
    if (s->start[i] < next_free)
      return fail(CHAIN_ERR_SHAPE, "%s: runs must ascend without overlap (run %d)", name, i);
    next_free = s->start[i] + s->len[i];
    if (next_free > INT32_MAX) return fail(CHAIN_ERR_UNSUPPORTED, "%s: positions beyond 2^31", name);
    total += s->len[i];
  }
  if (total != rows)
    return fail(CHAIN_ERR_SHAPE, "%s: runs cover %lld rows, tensor has %lld", name, (long long)total,
                (long long)rows);
  return CHAIN_OK;
}

#define TRY(x)                        \
  do {                                \
    chain_status s_ = (x);            \
    if (s_ != CHAIN_OK) return s_;    \
  } while (0)

// Shared validation of Q/K/V/O/LSE for both attention entry points.
chain_status check_attn(const chain_tensor *Q, const chain_tensor *K, const chain_tensor *V,
                        const chain_tensor *O, const chain_tensor *L, float scale, bool partial) {
  TRY(check_tensor(Q, "Q", 4));
  TRY(check_tensor(K, partial ? "Kc" : "K", 4));
  TRY(check_tensor(V, partial ? "Vc" : "V", 4));
  TRY(check_tensor(O, partial ? "O_part" : "O", 4));
  TRY(check_tensor(L, partial ? "LSE_part" : "LSE", 3, 4));
  if (K->dtype != Q->dtype || V->dtype != Q->dtype)
    return fail(CHAIN_ERR_DTYPE, "Q, K and V must share one dtype");
  if (partial ? O->dtype != CHAIN_F32 : O->dtype != Q->dtype)
    return fail(CHAIN_ERR_DTYPE, partial ? "O_part must be f32" : "O must have the dtype of Q");
  if (L->dtype != CHAIN_F32) return fail(CHAIN_ERR_DTYPE, "LSE must be f32");
  const int64_t B = Q->shape[0], Hq = Q->shape[1], Sq = Q->shape[2], D = Q->shape[3];
  for (int i = 0; i < 4; ++i)
    if (K->shape[i] != V->shape[i]) return fail(CHAIN_ERR_SHAPE, "K and V shapes differ");
  if (K->shape[0] != B || K->shape[3] != D) return fail(CHAIN_ERR_SHAPE, "K/V batch or head_dim differ from Q");
  for (int i = 0; i < 4; ++i)
    if (O->shape[i] != Q->shape[i]) return fail(CHAIN_ERR_SHAPE, "O shape must equal Q shape");
  if (L->shape[0] != B || L->shape[1] != Hq || L->shape[2] != Sq)
    return fail(CHAIN_ERR_SHAPE, "LSE shape must be [B, Hq, Sq]");
  const int64_t Hkv = K->shape[1];
  if (Hkv == 0 ? Hq != 0 : Hq % Hkv != 0)
    return fail(CHAIN_ERR_SHAPE, "query heads (%lld) must be a multiple of key/value heads (%lld)",
                (long long)Hq, (long long)Hkv);
  if (D != 64 && D != 128) return fail(CHAIN_ERR_UNSUPPORTED, "head_dim %lld (supported: 64, 128)", (long long)D);
  if (Sq > INT32_MAX / 2 || K->shape[2] > INT32_MAX / 2 || B * Hq > INT32_MAX)
    return fail(CHAIN_ERR_UNSUPPORTED, "sizes beyond 2^30 rows");
  // The bf16 kernels address one head's key/value rows with 32-bit byte offsets.
  if (Q->dtype == CHAIN_BF16 && K->shape[2] > 0) {
    const int64_t last = K->shape[2] - 1;
    if ((last * K->stride[2] + D) * 2 > INT32_MAX || (last * V->stride[2] + D) * 2 > INT32_MAX)
      return fail(CHAIN_ERR_UNSUPPORTED, "the key/value rows of one head span 2 GiB or more");
  }
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(CHAIN_ERR_UNSUPPORTED, "scale must be positive and finite");
  if (overlap(*O, *Q) || overlap(*O, *K) || overlap(*O, *V) || overlap(*L, *Q) || overlap(*L, *K) ||
      overlap(*L, *V) || overlap(*L, *O))
    return fail(CHAIN_ERR_ALIAS, "outputs overlap inputs or each other");
  return CHAIN_OK;
}

chain::AttnParams attn_params(const chain_tensor *Q, const chain_tensor *K, const chain_tensor *V,
                              const chain_tensor *O, const chain_tensor *L, int causal, float scale,
                              bool o_f32) {
  chain::AttnParams p;
  std::memset(&p, 0, sizeof p);
  p.q = Q->data;
  p.k = K->data;
  p.v = V->data;
  p.o = O->data;
  p.lse = (float *)L->data;
  p.q_sb = Q->stride[0], p.q_sh = Q->stride[1], p.q_ss = Q->stride[2];
  p.k_sb = K->stride[0], p.k_sh = K->stride[1], p.k_ss = K->stride[2];
  p.v_sb = V->stride[0], p.v_sh = V->stride[1], p.v_ss = V->stride[2];
  p.o_sb = O->stride[0], p.o_sh = O->stride[1], p.o_ss = O->stride[2];
  p.l_sb = L->stride[0], p.l_sh = L->stride[1], p.l_ss = L->stride[2];
  p.B = (int32_t)Q->shape[0];
  p.Hq = (int32_t)Q->shape[1];
  p.Hkv = (int32_t)K->shape[1];
  p.Sq = (int32_t)Q->shape[2];
  p.Sk = (int32_t)K->shape[2];
  p.causal = causal ? 1 : 0;
  p.o_f32 = o_f32 ? 1 : 0;
  p.scale_log2 = scale * 1.4426950408889634f;
  return p;
}

chain_status launch_attn(const chain::AttnParams &p, int D, int dtype, void *stream) {
  if (p.B == 0 || p.Hq == 0 || p.Sq == 0) return ok();
  hipError_t e = dtype == CHAIN_BF16 ? chain::launch_attn_mfma_bf16(p, D, (hipStream_t)stream)
                                     : chain::launch_attn_valu(p, D, dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(CHAIN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int chain_version(void) { return CHAIN_VERSION; }

const char *chain_status_str(chain_status s) {
  switch (s) {
    case CHAIN_OK: return "CHAIN_OK";
    case CHAIN_ERR_NULL: return "CHAIN_ERR_NULL";
    case CHAIN_ERR_DTYPE: return "CHAIN_ERR_DTYPE";
    case CHAIN_ERR_SHAPE: return "CHAIN_ERR_SHAPE";
    case CHAIN_ERR_LAYOUT: return "CHAIN_ERR_LAYOUT";
    case CHAIN_ERR_ALIGN: return "CHAIN_ERR_ALIGN";
    case CHAIN_ERR_ALIAS: return "CHAIN_ERR_ALIAS";
    case CHAIN_ERR_UNSUPPORTED: return "CHAIN_ERR_UNSUPPORTED";
    case CHAIN_ERR_WORKSPACE: return "CHAIN_ERR_WORKSPACE";
    case CHAIN_ERR_HIP: return "CHAIN_ERR_HIP";
  }
  return "CHAIN_ERR_UNKNOWN";
}

const char *chain_last_error(void) { return g_last_error.c_str(); }

chain_status chain_attn_fwd(const chain_tensor *Q, const chain_tensor *K, const chain_tensor *V,
                            const chain_tensor *O, const chain_tensor *LSE, int causal, float scale,
                            int n_chunks, int zigzag, void *stream) {
  TRY(check_attn(Q, K, V, O, LSE, scale, false));
  const int64_t S = Q->shape[2], Sk = K->shape[2];
  if (causal && Sk != S) return fail(CHAIN_ERR_SHAPE, "causal attention needs as many keys as queries");
  if (n_chunks < 1 || n_chunks > CHAIN_MAX_CHUNKS)
    return fail(CHAIN_ERR_SHAPE, "n_chunks %d outside 1..%d", n_chunks, CHAIN_MAX_CHUNKS);
  const int64_t pieces = zigzag ? 2 * (int64_t)n_chunks : n_chunks;
  if (Sk % pieces) return fail(CHAIN_ERR_SHAPE, "%lld keys do not split into %lld equal pieces", (long long)Sk, (long long)pieces);
  chain::AttnParams p = attn_params(Q, K, V, O, LSE, causal, scale, Q->dtype == CHAIN_F32);
  chain::build_row_runs(nullptr, S, &p.qruns);
  chain::build_fused_ranges(Sk, n_chunks, zigzag, &p.kr);
  return launch_attn(p, (int)Q->shape[3], Q->dtype, stream);
}

chain_status chain_attn_partial(const chain_tensor *Q, const chain_tensor *Kc, const chain_tensor *Vc,
                                const chain_tensor *O_part, const chain_tensor *LSE_part, int causal,
                                float scale, const chain_segs *q_pos, const chain_segs *kv_pos,
                                void *stream) {
  TRY(check_attn(Q, Kc, Vc, O_part, LSE_part, scale, true));
  TRY(check_segs(q_pos, Q->shape[2], "q_pos"));
  TRY(check_segs(kv_pos, Kc->shape[2], "kv_pos"));
  chain::AttnParams p = attn_params(Q, Kc, Vc, O_part, LSE_part, causal, scale, true);
  chain::build_row_runs(q_pos, Q->shape[2], &p.qruns);
  chain::build_run_ranges(*kv_pos, &p.kr);
  return launch_attn(p, (int)Q->shape[3], Q->dtype, stream);
}

chain_status chain_lse_merge(const chain_tensor *O_parts, const chain_tensor *LSE_parts,
                             const chain_tensor *O, const chain_tensor *LSE, void *stream) {
  TRY(check_tensor(O_parts, "O_parts", 5));
  TRY(check_tensor(LSE_parts, "LSE_parts", 4, 4));
  TRY(check_tensor(O, "O", 4, O && O->dtype == CHAIN_F32 ? 16 : 8));
  if (LSE) TRY(check_tensor(LSE, "LSE", 3, 4));
  if (O_parts->dtype != CHAIN_F32 || LSE_parts->dtype != CHAIN_F32)
    return fail(CHAIN_ERR_DTYPE, "partials must be f32");
  if (LSE && LSE->dtype != CHAIN_F32) return fail(CHAIN_ERR_DTYPE, "LSE must be f32");
  const int64_t C = O_parts->shape[0];
  for (int i = 0; i < 4; ++i) {
    if (LSE_parts->shape[i] != O_parts->shape[i]) return fail(CHAIN_ERR_SHAPE, "LSE_parts must be O_parts without D");
    if (O->shape[i] != O_parts->shape[i + 1]) return fail(CHAIN_ERR_SHAPE, "O must be O_parts without C");
  }
  if (LSE)
    for (int i = 0; i < 3; ++i)
      if (LSE->shape[i] != O_parts->shape[i + 1]) return fail(CHAIN_ERR_SHAPE, "LSE must be [B, H, S]");
  const int64_t D = O->shape[3];
  if (C < 1 || C > 64) return fail(CHAIN_ERR_SHAPE, "part count %lld outside 1..64", (long long)C);
  if (D % 4 || D > 256 || D == 0) return fail(CHAIN_ERR_UNSUPPORTED, "head_dim %lld (multiple of 4, <= 256)", (long long)D);
  if (overlap(*O, *O_parts) || overlap(*O, *LSE_parts) ||
      (LSE && (overlap(*LSE, *O_parts) || overlap(*LSE, *LSE_parts) || overlap(*LSE, *O))))
    return fail(CHAIN_ERR_ALIAS, "outputs overlap inputs or each other");
  const int64_t rows = O->shape[0] * O->shape[1] * O->shape[2];
  if (rows == 0) return ok();
  // the kernels index (batch, head) and row blocks of at least 8 rows by 32-bit
  // workgroup numbers, and rows by 32-bit positions
  const int64_t bh = O->shape[0] * O->shape[1], S = O->shape[2];
  if (S > INT32_MAX || bh > INT32_MAX || bh * ((S + 7) / 8) > INT32_MAX)
    return fail(CHAIN_ERR_UNSUPPORTED, "too many rows: %lld (batch, head) pairs of %lld rows",
                (long long)bh, (long long)S);
  chain::MergeParams p;
  std::memset(&p, 0, sizeof p);
  p.o_parts = (const float *)O_parts->data;
  p.lse_parts = (const float *)LSE_parts->data;
  p.o = O->data;
  p.lse = LSE ? (float *)LSE->data : nullptr;
  p.p_sc = O_parts->stride[0], p.p_sb = O_parts->stride[1], p.p_sh = O_parts->stride[2], p.p_ss = O_parts->stride[3];
  p.lp_sc = LSE_parts->stride[0], p.lp_sb = LSE_parts->stride[1], p.lp_sh = LSE_parts->stride[2], p.lp_ss = LSE_parts->stride[3];
  p.o_sb = O->stride[0], p.o_sh = O->stride[1], p.o_ss = O->stride[2];
  if (LSE) p.l_sb = LSE->stride[0], p.l_sh = LSE->stride[1], p.l_ss = LSE->stride[2];
  p.C = (int32_t)C;
  p.B = (int32_t)O->shape[0];
  p.H = (int32_t)O->shape[1];
  p.S = (int32_t)O->shape[2];
  p.D = (int32_t)D;
  p.o_f32 = O->dtype == CHAIN_F32;
  hipError_t e = chain::launch_lse_merge(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(CHAIN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

size_t chain_mlp_workspace_bytes(int64_t M, int64_t N, int32_t dt) {
  const size_t es = elem_size(dt);
  if (es == 0 || M < 0 || N < 0) return 0;
  const size_t b = (size_t)M * (size_t)N * es;
  return (b + 255) / 256 * 256;
}

}  // extern "C"

namespace {

// Device scratch of chain_mlp_fwd_noalloc: one copy per GPU, held until the
// process ends.  Host code never uses the array's name as an address (on the
// host it names a stand-in, not device memory); it uses the device address
// hipGetSymbolAddress returns for the current device, fetched once per device.
__device__ __align__(256) unsigned char scratch[CHAIN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

chain_status scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CHAIN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(CHAIN_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(CHAIN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return CHAIN_OK;
}

// chain_mlp_fwd's body.  With noalloc the caller's workspace arguments are
// ignored: H goes to this device's static scratch, and shapes whose H does not
// fit it are refused before anything else happens.
chain_status mlp_fwd_impl(const chain_tensor *X, const chain_tensor *W1, const chain_tensor *W2,
                          const chain_tensor *O, int act, void *workspace, size_t ws_bytes,
                          void *stream, bool noalloc) {
  TRY(check_tensor(X, "X", 2));
  TRY(check_tensor(W1, "W1", 2, 16, true));
  TRY(check_tensor(W2, "W2", 2, 16, true));
  TRY(check_tensor(O, "O", 2, O && O->dtype == CHAIN_F32 ? 4 : 2));
  if (W1->dtype != X->dtype || W2->dtype != X->dtype)
    return fail(CHAIN_ERR_DTYPE, "X, W1 and W2 must share one dtype");
  if (act != CHAIN_ACT_GELU_ERF && act != CHAIN_ACT_GELU_TANH && act != CHAIN_ACT_IDENTITY && act != CHAIN_ACT_SILU)
    return fail(CHAIN_ERR_UNSUPPORTED, "unknown activation %d", act);
  const int64_t M = X->shape[0], K = X->shape[1], N = W1->shape[1], K2 = W2->shape[1];
  if (W1->shape[0] != K || W2->shape[0] != N || O->shape[0] != M || O->shape[1] != K2)
    return fail(CHAIN_ERR_SHAPE, "expected X[M,K] W1[K,N] W2[N,K2] O[M,K2]");
  if (K % 8 || N % 8 || K2 % 8) return fail(CHAIN_ERR_UNSUPPORTED, "K, N and K2 must be multiples of 8");
  if (M > INT32_MAX || K > INT32_MAX || N > INT32_MAX || K2 > INT32_MAX)
    return fail(CHAIN_ERR_UNSUPPORTED, "sizes beyond 2^31");
  if (overlap(*O, *X) || overlap(*O, *W1) || overlap(*O, *W2))
    return fail(CHAIN_ERR_ALIAS, "O overlaps an input");
  const size_t need = chain_mlp_workspace_bytes(M, N, X->dtype);
  if (noalloc && need > CHAIN_NOALLOC_SCRATCH_BYTES)
    return fail(CHAIN_ERR_WORKSPACE, "H of %lld x %lld needs %zu bytes; the static scratch holds %zu",
                (long long)M, (long long)N, need, (size_t)CHAIN_NOALLOC_SCRATCH_BYTES);
  if (M == 0 || K2 == 0) return ok();
  if (noalloc) {
    TRY(scratch_address(&workspace));
    ws_bytes = CHAIN_NOALLOC_SCRATCH_BYTES;
  }
  if (workspace == nullptr || ws_bytes < need)
    return fail(CHAIN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  if ((uintptr_t)workspace % 256) return fail(CHAIN_ERR_ALIGN, "workspace must be 256-byte aligned");
  {
    chain_tensor H{};
    H.data = workspace;
    H.dtype = X->dtype;
    H.ndim = 2;
    H.shape[0] = M, H.shape[1] = N;
    H.stride[0] = N, H.stride[1] = 1;
    if (overlap(H, *X) || overlap(H, *W1) || overlap(H, *W2) || overlap(H, *O))
      return fail(CHAIN_ERR_ALIAS, "workspace overlaps a tensor");
  }
  // B strides: element (k, n) at b[k * b_sk + n * b_sn].  With one of the
  // two extents 1 its stride is arbitrary; pick the layout the other implies.
  auto b_strides = [](const chain_tensor &w, chain::GemmParams &g) {
    const bool kmajor = !(w.shape[1] <= 1 || w.stride[1] == 1);
    g.b_sk = kmajor ? 1 : (w.shape[0] <= 1 ? w.shape[1] : w.stride[0]);
    g.b_sn = kmajor ? w.stride[1] : 1;
  };
  const size_t es = elem_size(X->dtype), oes = elem_size(O->dtype);
  chain::GemmParams g1{}, g2{};
  g1.a = X->data, g1.b = W1->data, g1.c = workspace;
  g1.lda = X->stride[0], g1.ldc = N;
  b_strides(*W1, g1);
  g1.M = (int32_t)M, g1.N = (int32_t)N, g1.K = (int32_t)K;
  g1.act = act;
  g1.c_f32 = X->dtype == CHAIN_F32;
  g1.c_vec = (N * es) % (4 * es) == 0;   // workspace is 256-byte aligned
  g2.a = workspace, g2.b = W2->data, g2.c = O->data;
  g2.lda = N, g2.ldc = O->stride[0];
  b_strides(*W2, g2);
  g2.M = (int32_t)M, g2.N = (int32_t)K2, g2.K = (int32_t)N;
  g2.act = CHAIN_ACT_IDENTITY;
  g2.c_f32 = O->dtype == CHAIN_F32;
  g2.c_vec = (uintptr_t)O->data % (4 * oes) == 0 && (M <= 1 || (O->stride[0] * oes) % (4 * oes) == 0);
  const int64_t kMaxStride = int64_t(1) << 25;   // per-thread offsets within a tile stay 32-bit
  for (const int64_t st : {g1.lda, g1.b_sk, g1.b_sn, g2.b_sk, g2.b_sn, g2.ldc})
    if (st > kMaxStride) return fail(CHAIN_ERR_UNSUPPORTED, "row strides beyond 2^25 elements");
  hipError_t e = chain::launch_gemm(g1, X->dtype, (hipStream_t)stream);
  if (e == hipSuccess) e = chain::launch_gemm(g2, X->dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(CHAIN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

chain_status chain_mlp_fwd(const chain_tensor *X, const chain_tensor *W1, const chain_tensor *W2,
                           const chain_tensor *O, int act, void *workspace, size_t ws_bytes,
                           void *stream) {
  return mlp_fwd_impl(X, W1, W2, O, act, workspace, ws_bytes, stream, false);
}

chain_status chain_mlp_fwd_noalloc(const chain_tensor *X, const chain_tensor *W1, const chain_tensor *W2,
                                   const chain_tensor *O, int act, void *stream) {
  return mlp_fwd_impl(X, W1, W2, O, act, nullptr, 0, stream, true);
}

size_t chain_attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t S) {
  if (B < 0 || Hq < 0 || S < 0) return 0;
  const size_t b = (size_t)B * (size_t)Hq * (size_t)((S + 63) / 64 * 64) * 8;
  return (b + 255) / 256 * 256;
}

chain_status chain_attn_bwd(const chain_tensor *Q, const chain_tensor *K, const chain_tensor *V,
                            const chain_tensor *O, const chain_tensor *LSE, const chain_tensor *dO,
                            const chain_tensor *dQ, const chain_tensor *dK, const chain_tensor *dV,
                            int causal, float scale, void *workspace, size_t ws_bytes, void *stream) {
  TRY(check_attn(Q, K, V, O, LSE, scale, false));
  TRY(check_tensor(dO, "dO", 4));
  TRY(check_tensor(dQ, "dQ", 4));
  TRY(check_tensor(dK, "dK", 4));
  TRY(check_tensor(dV, "dV", 4));
  if (Q->dtype != CHAIN_BF16 || dO->dtype != CHAIN_BF16)
    return fail(CHAIN_ERR_DTYPE, "Q, K, V, O and dO must be bf16");
  if (dQ->dtype != CHAIN_F32 || dK->dtype != CHAIN_F32 || dV->dtype != CHAIN_F32)
    return fail(CHAIN_ERR_DTYPE, "dQ, dK and dV must be f32");
  const int64_t B = Q->shape[0], Hq = Q->shape[1], S = Q->shape[2], D = Q->shape[3];
  if (K->shape[2] != S) return fail(CHAIN_ERR_SHAPE, "the backward needs as many keys as queries");
  for (int i = 0; i < 4; ++i) {
    if (dO->shape[i] != Q->shape[i] || dQ->shape[i] != Q->shape[i])
      return fail(CHAIN_ERR_SHAPE, "dO and dQ must have the shape of Q");
    if (dK->shape[i] != K->shape[i] || dV->shape[i] != K->shape[i])
      return fail(CHAIN_ERR_SHAPE, "dK and dV must have the shape of K");
  }
  if (B * Hq * S > INT32_MAX) return fail(CHAIN_ERR_UNSUPPORTED, "B * Hq * S beyond 2^31");
  // The kernels address one head's query and dO rows with 32-bit byte offsets.
  if (S > 0 && (((S - 1) * Q->stride[2] + D) * 2 > INT32_MAX || ((S - 1) * dO->stride[2] + D) * 2 > INT32_MAX))
    return fail(CHAIN_ERR_UNSUPPORTED, "the query or dO rows of one head span 2 GiB or more");
  const chain_tensor *ins[] = {Q, K, V, O, LSE, dO};
  const chain_tensor *outs[] = {dQ, dK, dV};
  for (int i = 0; i < 3; ++i) {
    for (const chain_tensor *t : ins)
      if (overlap(*outs[i], *t)) return fail(CHAIN_ERR_ALIAS, "outputs overlap inputs or each other");
    for (int j = 0; j < i; ++j)
      if (overlap(*outs[i], *outs[j])) return fail(CHAIN_ERR_ALIAS, "outputs overlap inputs or each other");
  }
  const size_t need = chain_attn_bwd_workspace_bytes(B, Hq, S);
  if (B == 0 || Hq == 0 || S == 0) return ok();
  if (workspace == nullptr || ws_bytes < need)
    return fail(CHAIN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  if ((uintptr_t)workspace % 256) return fail(CHAIN_ERR_ALIGN, "workspace must be 256-byte aligned");
  {
    chain_tensor W{};
    W.data = workspace;
    W.dtype = CHAIN_F32;
    W.ndim = 1;
    W.shape[0] = (int64_t)(need / 4);
    W.stride[0] = 1;
    for (const chain_tensor *t : ins)
      if (overlap(W, *t)) return fail(CHAIN_ERR_ALIAS, "workspace overlaps a tensor");
    for (const chain_tensor *t : outs)
      if (overlap(W, *t)) return fail(CHAIN_ERR_ALIAS, "workspace overlaps a tensor");
  }
  chain::AttnBwdParams p;
  std::memset(&p, 0, sizeof p);
  p.q = Q->data, p.k = K->data, p.v = V->data, p.o = O->data, p.dout = dO->data;
  p.lse = (const float *)LSE->data;
  p.dq = (float *)dQ->data, p.dk = (float *)dK->data, p.dv = (float *)dV->data;
  p.rowv = (float *)workspace;
  p.q_sb = Q->stride[0], p.q_sh = Q->stride[1], p.q_ss = Q->stride[2];
  p.k_sb = K->stride[0], p.k_sh = K->stride[1], p.k_ss = K->stride[2];
  p.v_sb = V->stride[0], p.v_sh = V->stride[1], p.v_ss = V->stride[2];
  p.o_sb = O->stride[0], p.o_sh = O->stride[1], p.o_ss = O->stride[2];
  p.do_sb = dO->stride[0], p.do_sh = dO->stride[1], p.do_ss = dO->stride[2];
  p.l_sb = LSE->stride[0], p.l_sh = LSE->stride[1], p.l_ss = LSE->stride[2];
  p.dq_sb = dQ->stride[0], p.dq_sh = dQ->stride[1], p.dq_ss = dQ->stride[2];
  p.dk_sb = dK->stride[0], p.dk_sh = dK->stride[1], p.dk_ss = dK->stride[2];
  p.dv_sb = dV->stride[0], p.dv_sh = dV->stride[1], p.dv_ss = dV->stride[2];
  p.B = (int32_t)B, p.Hq = (int32_t)Hq, p.Hkv = (int32_t)K->shape[1], p.S = (int32_t)S;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = chain::launch_attn_bwd(p, (int)D, (hipStream_t)stream);
  if (e != hipSuccess) return fail(CHAIN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

chain_status chain_mlp_gated_fwd(const chain_tensor *X, const chain_tensor *Wg, const chain_tensor *Wu,
                                 const chain_tensor *Wd, const chain_tensor *O, int act, void *workspace,
                                 size_t ws_bytes, void *stream) {
  TRY(check_tensor(X, "X", 2));
  TRY(check_tensor(Wg, "Wg", 2, 16, true));
  TRY(check_tensor(Wu, "Wu", 2, 16, true));
  TRY(check_tensor(Wd, "Wd", 2, 16, true));
  TRY(check_tensor(O, "O", 2, O && O->dtype == CHAIN_F32 ? 4 : 2));
  if (Wg->dtype != X->dtype || Wu->dtype != X->dtype || Wd->dtype != X->dtype)
    return fail(CHAIN_ERR_DTYPE, "X, Wg, Wu and Wd must share one dtype");
  if (act != CHAIN_ACT_GELU_ERF && act != CHAIN_ACT_GELU_TANH && act != CHAIN_ACT_IDENTITY && act != CHAIN_ACT_SILU)
    return fail(CHAIN_ERR_UNSUPPORTED, "unknown activation %d", act);
  const int64_t M = X->shape[0], K = X->shape[1], N = Wg->shape[1], K2 = Wd->shape[1];
  if (Wg->shape[0] != K || Wu->shape[0] != K || Wu->shape[1] != N || Wd->shape[0] != N ||
      O->shape[0] != M || O->shape[1] != K2)
    return fail(CHAIN_ERR_SHAPE, "expected X[M,K] Wg[K,N] Wu[K,N] Wd[N,K2] O[M,K2]");
  if (X->dtype != CHAIN_BF16) return fail(CHAIN_ERR_UNSUPPORTED, "the gated form takes bf16 inputs");
  if (K % 8 || N % 8 || K2 % 8) return fail(CHAIN_ERR_UNSUPPORTED, "K, N and K2 must be multiples of 8");
  if (M > INT32_MAX || K > INT32_MAX || N > INT32_MAX || K2 > INT32_MAX)
    return fail(CHAIN_ERR_UNSUPPORTED, "sizes beyond 2^31");
  // Gate and up weights: one layout and one stride for both, k contiguous
  // (column-major) or n contiguous (row-major).
  auto kmajor = [](const chain_tensor &w) { return w.shape[0] <= 1 || w.stride[0] == 1; };
  auto nmajor = [](const chain_tensor &w) { return w.shape[1] <= 1 || w.stride[1] == 1; };
  const int64_t gsn = Wg->shape[1] <= 1 ? K : Wg->stride[1], usn = Wu->shape[1] <= 1 ? K : Wu->stride[1];
  const int64_t gsk = Wg->shape[0] <= 1 ? N : Wg->stride[0], usk = Wu->shape[0] <= 1 ? N : Wu->stride[0];
  const bool gu_k = kmajor(*Wg) && kmajor(*Wu) && gsn == usn;
  const bool gu_n = !gu_k && nmajor(*Wg) && nmajor(*Wu) && gsk == usk;
  if (K > 0 && N > 0 && !gu_k && !gu_n)
    return fail(CHAIN_ERR_UNSUPPORTED, "gate and up weights must share one layout (row- or column-major) and strides");
  if (overlap(*O, *X) || overlap(*O, *Wg) || overlap(*O, *Wu) || overlap(*O, *Wd))
    return fail(CHAIN_ERR_ALIAS, "O overlaps an input");
  const size_t need = chain_mlp_workspace_bytes(M, N, CHAIN_BF16);
  if (M == 0 || K2 == 0) return ok();
  if (workspace == nullptr || ws_bytes < need)
    return fail(CHAIN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  if ((uintptr_t)workspace % 256) return fail(CHAIN_ERR_ALIGN, "workspace must be 256-byte aligned");
  {
    chain_tensor H{};
    H.data = workspace;
    H.dtype = CHAIN_BF16;
    H.ndim = 2;
    H.shape[0] = M, H.shape[1] = N;
    H.stride[0] = N, H.stride[1] = 1;
    if (overlap(H, *X) || overlap(H, *Wg) || overlap(H, *Wu) || overlap(H, *Wd) || overlap(H, *O))
      return fail(CHAIN_ERR_ALIAS, "workspace overlaps a tensor");
  }
  const size_t oes = elem_size(O->dtype);
  chain::GemmParams g1{}, g2{};
  g1.a = X->data, g1.b = Wg->data, g1.b2 = Wu->data, g1.gated = 1, g1.c = workspace;
  g1.lda = X->stride[0], g1.ldc = N;
  if (gu_n) g1.b_sk = gsk, g1.b_sn = 1;
  else g1.b_sk = 1, g1.b_sn = gsn;
  g1.M = (int32_t)M, g1.N = (int32_t)N, g1.K = (int32_t)K;
  g1.act = act;
  g1.c_f32 = 0;
  g1.c_vec = N % 4 == 0;   // workspace is 256-byte aligned
  g2.a = workspace, g2.b = Wd->data, g2.c = O->data;
  g2.lda = N, g2.ldc = O->stride[0];
  const bool dk = !(Wd->shape[1] <= 1 || Wd->stride[1] == 1);
  g2.b_sk = dk ? 1 : (Wd->shape[0] <= 1 ? Wd->shape[1] : Wd->stride[0]);
  g2.b_sn = dk ? Wd->stride[1] : 1;
  g2.M = (int32_t)M, g2.N = (int32_t)K2, g2.K = (int32_t)N;
  g2.act = CHAIN_ACT_IDENTITY;
  g2.c_f32 = O->dtype == CHAIN_F32;
  g2.c_vec = (uintptr_t)O->data % (4 * oes) == 0 && (M <= 1 || (O->stride[0] * oes) % (4 * oes) == 0);
  const int64_t kMaxStride = int64_t(1) << 25;   // per-thread offsets within a tile stay 32-bit
  for (const int64_t st : {g1.lda, g1.b_sk, g1.b_sn, g2.b_sk, g2.b_sn, g2.ldc})
    if (st > kMaxStride) return fail(CHAIN_ERR_UNSUPPORTED, "row strides beyond 2^25 elements");
  if (gu_n && N > 0 && K > 0 && !chain::gemm_gated_rowmajor_ok(g1))
    return fail(CHAIN_ERR_UNSUPPORTED, "row-major gate and up weights: rows beyond 32-bit offsets");
  hipError_t e = hipSuccess;
  if (N > 0) e = chain::launch_gemm(g1, CHAIN_BF16, (hipStream_t)stream);
  if (e == hipSuccess) e = chain::launch_gemm(g2, CHAIN_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return fail(CHAIN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

size_t chain_linear_attn_workspace_bytes(int64_t B, int64_t Hkv, int64_t S, int64_t D) {
  if (B < 0 || Hkv < 0 || S < 0 || D < 0) return 0;
  return chain::linear_attn_workspace_bytes(B, Hkv, S, D);
}

chain_status chain_linear_attn_fwd(const chain_tensor *Q, const chain_tensor *K, const chain_tensor *V,
                                   const chain_tensor *O, const chain_tensor *S_in, const chain_tensor *S_out,
                                   void *workspace, size_t ws_bytes, void *stream) {
  TRY(check_tensor(Q, "Q", 4));
  TRY(check_tensor(K, "K", 4));
  TRY(check_tensor(V, "V", 4));
  TRY(check_tensor(O, "O", 4));
  if (S_in) TRY(check_tensor(S_in, "S_in", 4, 4));
  if (S_out) TRY(check_tensor(S_out, "S_out", 4, 4));
  if (Q->dtype != CHAIN_BF16 || K->dtype != CHAIN_BF16 || V->dtype != CHAIN_BF16)
    return fail(CHAIN_ERR_DTYPE, "Q, K and V must be bf16");
  if ((S_in && S_in->dtype != CHAIN_F32) || (S_out && S_out->dtype != CHAIN_F32))
    return fail(CHAIN_ERR_DTYPE, "states must be f32");
  const int64_t B = Q->shape[0], Hq = Q->shape[1], S = Q->shape[2], D = Q->shape[3];
  for (int i = 0; i < 4; ++i) {
    if (K->shape[i] != V->shape[i]) return fail(CHAIN_ERR_SHAPE, "K and V shapes differ");
    if (O->shape[i] != Q->shape[i]) return fail(CHAIN_ERR_SHAPE, "O shape must equal Q shape");
  }
  if (K->shape[0] != B || K->shape[2] != S || K->shape[3] != D)
    return fail(CHAIN_ERR_SHAPE, "K/V must be [B, Hkv, S, D] with Q's B, S and D");
  const int64_t Hkv = K->shape[1];
  if (Hkv == 0 ? Hq != 0 : Hq % Hkv != 0)
    return fail(CHAIN_ERR_SHAPE, "query heads must be a multiple of key/value heads");
  for (const chain_tensor *st : {S_in, S_out})
    if (st && (st->shape[0] != B || st->shape[1] != Hkv || st->shape[2] != D || st->shape[3] != D))
      return fail(CHAIN_ERR_SHAPE, "states must be [B, Hkv, D, D]");
  if (D != 64 && D != 128) return fail(CHAIN_ERR_UNSUPPORTED, "head_dim %lld (supported: 64, 128)", (long long)D);
  if (S > INT32_MAX / 2 || B * Hq * ((S + 127) / 128) > INT32_MAX || B * Hkv * 16 > INT32_MAX)
    return fail(CHAIN_ERR_UNSUPPORTED, "sizes too large");
  const chain_tensor *ins[] = {Q, K, V, S_in};
  for (const chain_tensor *t : ins)
    if (t && (overlap(*O, *t) || (S_out && overlap(*S_out, *t))))
      return fail(CHAIN_ERR_ALIAS, "outputs overlap inputs or each other");
  if (S_out && overlap(*S_out, *O)) return fail(CHAIN_ERR_ALIAS, "outputs overlap inputs or each other");
  if (B == 0 || Hkv == 0) return ok();
  const size_t need = chain::linear_attn_workspace_bytes(B, Hkv, S, D);
  if (S > 0) {
    if (workspace == nullptr || ws_bytes < need)
      return fail(CHAIN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
    if ((uintptr_t)workspace % 256) return fail(CHAIN_ERR_ALIGN, "workspace must be 256-byte aligned");
    chain_tensor W{};
    W.data = workspace;
    W.dtype = CHAIN_F32;
    W.ndim = 1;
    W.shape[0] = (int64_t)(need / 4);
    W.stride[0] = 1;
    for (const chain_tensor *t : {Q, K, V, O, S_in, S_out})
      if (t && overlap(W, *t)) return fail(CHAIN_ERR_ALIAS, "workspace overlaps a tensor");
  }
  chain::LinAttnParams p;
  std::memset(&p, 0, sizeof p);
  p.q = Q->data, p.k = K->data, p.v = V->data, p.o = O->data;
  p.s_in = S_in ? (const float *)S_in->data : nullptr;
  p.s_out = S_out ? (float *)S_out->data : nullptr;
  if (workspace) {
    size_t off[3];
    chain::linear_attn_workspace_layout(B, Hkv, S, D, off);
    p.sub_total = (float *)((char *)workspace + off[0]);
    p.seg_base = (float *)((char *)workspace + off[1]);
  }
  p.q_sb = Q->stride[0], p.q_sh = Q->stride[1], p.q_ss = Q->stride[2];
  p.k_sb = K->stride[0], p.k_sh = K->stride[1], p.k_ss = K->stride[2];
  p.v_sb = V->stride[0], p.v_sh = V->stride[1], p.v_ss = V->stride[2];
  p.o_sb = O->stride[0], p.o_sh = O->stride[1], p.o_ss = O->stride[2];
  if (S_in) p.si_sb = S_in->stride[0], p.si_sh = S_in->stride[1], p.si_sr = S_in->stride[2];
  if (S_out) p.so_sb = S_out->stride[0], p.so_sh = S_out->stride[1], p.so_sr = S_out->stride[2];
  p.B = (int32_t)B, p.Hq = (int32_t)Hq, p.Hkv = (int32_t)Hkv, p.S = (int32_t)S;
  p.o_f32 = O->dtype == CHAIN_F32;
  hipError_t e = chain::launch_linear_attn(p, (int)D, (hipStream_t)stream);
  if (e != hipSuccess) return fail(CHAIN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

chain_status chain_zigzag_segs(int64_t S, int32_t parts, int32_t r, chain_segs *out) {
  if (out == nullptr) return fail(CHAIN_ERR_NULL, "out is NULL");
  if (parts < 1 || S <= 0 || S % (2 * (int64_t)parts))
    return fail(CHAIN_ERR_SHAPE, "%lld tokens do not split into %d zigzag pieces", (long long)S, 2 * parts);
  if (r < 0 || r >= parts) return fail(CHAIN_ERR_SHAPE, "share %d outside 0..%d", r, parts - 1);
  const int64_t n = S / (2 * (int64_t)parts);
  std::memset(out, 0, sizeof *out);
  out->n = 2;
  out->start[0] = r * n;
  out->len[0] = n;
  out->start[1] = (2 * (int64_t)parts - 1 - r) * n;
  out->len[1] = n;
  return ok();
}

chain_status chain_attn_tile_census(int64_t Sq, const chain_segs *q_pos, int64_t Sk,
                                    const chain_segs *kv_pos, int n_chunks, int zigzag, int causal,
                                    int block_m, int block_n, int64_t *full, int64_t *diag,
                                    int64_t *skip) {
  if (!full || !diag || !skip) return fail(CHAIN_ERR_NULL, "count pointers must not be NULL");
  if (block_m < 1 || block_n < 1 || Sq < 0 || Sk < 0) return fail(CHAIN_ERR_SHAPE, "bad sizes");
  if (Sq > INT32_MAX / 2 || Sk > INT32_MAX / 2) return fail(CHAIN_ERR_UNSUPPORTED, "sizes beyond 2^30");
  if (q_pos) TRY(check_segs(q_pos, Sq, "q_pos"));
  chain::RowRuns rr;
  chain::build_row_runs(q_pos, Sq, &rr);
  chain::KeyRanges kr;
  if (kv_pos) {
    TRY(check_segs(kv_pos, Sk, "kv_pos"));
    chain::build_run_ranges(*kv_pos, &kr);
  } else {
    if (n_chunks < 1 || n_chunks > CHAIN_MAX_CHUNKS) return fail(CHAIN_ERR_SHAPE, "bad n_chunks");
    const int64_t pieces = zigzag ? 2 * (int64_t)n_chunks : n_chunks;
    if (Sk % pieces) return fail(CHAIN_ERR_SHAPE, "keys do not split into equal pieces");
    chain::build_fused_ranges(Sk, n_chunks, zigzag, &kr);
  }
  *full = *diag = *skip = 0;
  for (int64_t r0 = 0; r0 < Sq; r0 += block_m) {
    const int64_t r1 = r0 + block_m < Sq ? r0 + block_m : Sq;
    const int32_t qmin = chain::row_position(rr, (int32_t)r0);
    const int32_t qmax = chain::row_position(rr, (int32_t)(r1 - 1));
    for (int i = 0; i < kr.n; ++i)
      for (int64_t k0 = kr.beg[i]; k0 < kr.end[i]; k0 += block_n) {
        const int64_t nvalid = kr.end[i] - k0 < block_n ? kr.end[i] - k0 : block_n;
        const int c = chain::classify_tile(causal, qmin, qmax, (int32_t)(k0 + kr.pos_off[i]),
                                           (int32_t)(k0 + nvalid - 1 + kr.pos_off[i]), nvalid < block_n);
        (c == chain::TILE_FULL ? *full : c == chain::TILE_DIAG ? *diag : *skip) += 1;
      }
  }
  return ok();
}

}  // extern "C"
