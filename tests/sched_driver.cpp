// Host-side driver for the sanitizer build of libchain's host code (test
// infrastructure).  Prints one JSON object per line: the zigzag segments, the
// fused key ranges, row positions of position runs, the XCD work-item remap,
// tile censuses, and the status of every entry point called with invalid
// arguments.  Descriptors carry fake, never-dereferenced device addresses, so
// nothing here touches a GPU.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "chain.h"
#include "internal.h"

namespace {

const uintptr_t kFake = 0x7F0000000000ull;

chain_tensor td(std::vector<int64_t> shape, int32_t dt, uintptr_t data, std::vector<int64_t> stride = {}) {
  chain_tensor t{};
  t.data = (void *)data;
  t.dtype = dt;
  t.ndim = (int32_t)shape.size();
  if (stride.empty()) {
    stride.assign(shape.size(), 1);
    for (int i = (int)shape.size() - 2; i >= 0; --i) stride[i] = stride[i + 1] * shape[i + 1];
  }
  for (size_t i = 0; i < shape.size(); ++i) {
    t.shape[i] = shape[i];
    t.stride[i] = stride[i];
  }
  return t;
}

void print_status(const char *name, int st) { printf("{\"call\": \"%s\", \"st\": %d}\n", name, st); }

}  // namespace

int main() {
  // zigzag shares: both runs, or the status of an invalid request
  const int zz[][2] = {{32, 1}, {256, 8}, {96, 3}, {32768, 8}, {65536, 16}, {768, 8}};
  for (auto &c : zz)
    for (int r = 0; r < c[1]; ++r) {
      chain_segs s{};
      const int st = chain_zigzag_segs(c[0], c[1], r, &s);
      printf("{\"zz\": [%d, %d, %d], \"st\": %d, \"runs\": [", c[0], c[1], r, st);
      for (int i = 0; i < s.n; ++i) printf("%s[%lld, %lld]", i ? ", " : "", (long long)s.start[i], (long long)s.len[i]);
      printf("]}\n");
    }
  {
    chain_segs s{};
    print_status("zigzag_uneven", chain_zigzag_segs(100, 3, 0, &s));
    print_status("zigzag_rank_out_of_range", chain_zigzag_segs(256, 8, 8, &s));
    print_status("zigzag_null", chain_zigzag_segs(256, 8, 0, nullptr));
  }

  // fused key ranges in visit order
  const int fr[][3] = {{256, 1, 0}, {256, 4, 1}, {1024, 16, 1}, {192, 3, 0}, {65536, 16, 1}, {640, 5, 1}};
  for (auto &c : fr) {
    chain::KeyRanges kr;
    chain::build_fused_ranges(c[0], c[1], c[2], &kr);
    printf("{\"fused\": [%d, %d, %d], \"ranges\": [", c[0], c[1], c[2]);
    for (int i = 0; i < kr.n; ++i) printf("%s[%d, %d, %d]", i ? ", " : "", kr.beg[i], kr.end[i], kr.pos_off[i]);
    printf("]}\n");
  }

  // position runs: positions of every row, and the key ranges of the same runs
  {
    chain_segs s{};
    s.n = 3;
    const int64_t st[3] = {5, 40, 100}, ln[3] = {7, 0, 20};
    for (int i = 0; i < 3; ++i) s.start[i] = st[i], s.len[i] = ln[i];
    chain::RowRuns rr;
    chain::build_row_runs(&s, 27, &rr);
    printf("{\"rowpos\": [[5, 7], [40, 0], [100, 20]], \"pos\": [");
    for (int r = 0; r < 27; ++r) printf("%s%d", r ? ", " : "", chain::row_position(rr, r));
    printf("]}\n");
    chain::KeyRanges kr;
    chain::build_run_ranges(s, &kr);
    printf("{\"runranges\": [[5, 7], [40, 0], [100, 20]], \"ranges\": [");
    for (int i = 0; i < kr.n; ++i) printf("%s[%d, %d, %d]", i ? ", " : "", kr.beg[i], kr.end[i], kr.pos_off[i]);
    printf("]}\n");
  }

  // XCD remap: a bijection of [0, n) for every n
  const int ns[] = {1, 2, 3, 7, 8, 9, 15, 16, 17, 255, 256, 257, 1000, 4096, 4097};
  for (int n : ns) {
    std::vector<int> seen(n, 0);
    bool ok = true;
    for (int b = 0; b < n; ++b) {
      const int x = chain::xcd_remap(b, n);
      if (x < 0 || x >= n || seen[x]++) ok = false;
    }
    printf("{\"xcd\": %d, \"ok\": %s}\n", n, ok ? "true" : "false");
  }

  // tile censuses of the fused schedule and of ring shares
  const int cs[][5] = {{256, 32, 64, 1, 0}, {256, 32, 64, 4, 1}, {300, 32, 64, 1, 0}, {512, 128, 64, 8, 1},
                       {1024, 32, 64, 16, 1}, {192, 32, 64, 3, 0}, {640, 64, 64, 5, 1}};
  for (auto &c : cs) {
    int64_t f = -1, d = -1, k = -1;
    const int st = chain_attn_tile_census(c[0], nullptr, c[0], nullptr, c[3], c[4], 1, c[1], c[2], &f, &d, &k);
    printf("{\"census\": [%d, %d, %d, %d, %d], \"st\": %d, \"counts\": [%lld, %lld, %lld]}\n", c[0], c[1], c[2],
           c[3], c[4], st, (long long)f, (long long)d, (long long)k);
  }
  for (int r = 0; r < 8; ++r)
    for (int s = 0; s < 8; ++s) {
      chain_segs q{}, kv{};
      chain_zigzag_segs(768, 8, r, &q);
      chain_zigzag_segs(768, 8, s, &kv);
      int64_t f = -1, d = -1, k = -1;
      const int st = chain_attn_tile_census(96, &q, 96, &kv, 1, 0, 1, 32, 64, &f, &d, &k);
      printf("{\"share_census\": [768, 8, %d, %d], \"st\": %d, \"counts\": [%lld, %lld, %lld]}\n", r, s, st,
             (long long)f, (long long)d, (long long)k);
    }

  // validation: every entry point with invalid arguments (no launch may happen)
  const int BF = CHAIN_BF16, F32 = CHAIN_F32;
  const uintptr_t G = 1ull << 30;
  chain_tensor Q = td({1, 4, 256, 64}, BF, kFake), K = td({1, 2, 256, 64}, BF, kFake + G),
               V = td({1, 2, 256, 64}, BF, kFake + 2 * G), O = td({1, 4, 256, 64}, BF, kFake + 3 * G),
               L = td({1, 4, 256}, F32, kFake + 4 * G);
  print_status("attn_null_q", chain_attn_fwd(nullptr, &K, &V, &O, &L, 1, 0.125f, 1, 0, nullptr));
  chain_tensor Kf = td({1, 2, 256, 64}, F32, kFake + G);
  print_status("attn_dtype", chain_attn_fwd(&Q, &Kf, &V, &O, &L, 1, 0.125f, 1, 0, nullptr));
  chain_tensor K3 = td({1, 3, 256, 64}, BF, kFake + G);
  print_status("attn_heads", chain_attn_fwd(&Q, &K3, &V, &O, &L, 1, 0.125f, 1, 0, nullptr));
  print_status("attn_chunks", chain_attn_fwd(&Q, &K, &V, &O, &L, 1, 0.125f, 3, 0, nullptr));
  print_status("attn_chunks_zigzag", chain_attn_fwd(&Q, &K, &V, &O, &L, 1, 0.125f, 3, 1, nullptr));
  print_status("attn_chunks_max", chain_attn_fwd(&Q, &K, &V, &O, &L, 1, 0.125f, CHAIN_MAX_CHUNKS + 1, 0, nullptr));
  chain_tensor Qa = td({1, 4, 256, 64}, BF, kFake + 8);
  print_status("attn_align", chain_attn_fwd(&Qa, &K, &V, &O, &L, 1, 0.125f, 1, 0, nullptr));
  chain_tensor Oal = td({1, 4, 256, 64}, BF, kFake + 64);
  print_status("attn_alias", chain_attn_fwd(&Q, &K, &V, &Oal, &L, 1, 0.125f, 1, 0, nullptr));
  chain_tensor Qt = td({1, 4, 256, 64}, BF, kFake, {65536, 16384, 1, 256});
  print_status("attn_layout", chain_attn_fwd(&Qt, &K, &V, &O, &L, 1, 0.125f, 1, 0, nullptr));
  chain_tensor Q96 = td({1, 4, 256, 96}, BF, kFake), K96 = td({1, 2, 256, 96}, BF, kFake + G),
               V96 = td({1, 2, 256, 96}, BF, kFake + 2 * G), O96 = td({1, 4, 256, 96}, BF, kFake + 3 * G);
  print_status("attn_headdim", chain_attn_fwd(&Q96, &K96, &V96, &O96, &L, 1, 0.125f, 1, 0, nullptr));
  print_status("attn_scale_nan", chain_attn_fwd(&Q, &K, &V, &O, &L, 1, 0.f / 0.f, 1, 0, nullptr));

  chain_segs qs{}, ks{};
  qs.n = 1, qs.start[0] = 0, qs.len[0] = 256;
  ks.n = 1, ks.start[0] = 0, ks.len[0] = 255;
  chain_tensor Op = td({1, 4, 256, 64}, F32, kFake + 3 * G);
  print_status("partial_kv_segs_cover", chain_attn_partial(&Q, &K, &V, &Op, &L, 1, 0.125f, &qs, &ks, nullptr));
  ks.len[0] = 256;
  chain_segs bad{};
  bad.n = 2, bad.start[0] = 10, bad.len[0] = 100, bad.start[1] = 50, bad.len[1] = 156;
  print_status("partial_q_segs_overlap", chain_attn_partial(&Q, &K, &V, &Op, &L, 1, 0.125f, &bad, &ks, nullptr));
  print_status("partial_o_dtype", chain_attn_partial(&Q, &K, &V, &O, &L, 1, 0.125f, &qs, &ks, nullptr));
  print_status("partial_null_segs", chain_attn_partial(&Q, &K, &V, &Op, &L, 1, 0.125f, nullptr, &ks, nullptr));

  chain_tensor Ops = td({8, 1, 4, 256, 64}, F32, kFake), Lps = td({8, 1, 4, 256}, F32, kFake + G),
               Lp7 = td({7, 1, 4, 256}, F32, kFake + G), Om = td({1, 4, 256, 64}, BF, kFake + 2 * G),
               Lm = td({1, 4, 256}, F32, kFake + 3 * G);
  print_status("merge_parts_mismatch", chain_lse_merge(&Ops, &Lp7, &Om, &Lm, nullptr));
  chain_tensor Omal = td({1, 4, 256, 64}, BF, kFake + 64);
  print_status("merge_alias", chain_lse_merge(&Ops, &Lps, &Omal, &Lm, nullptr));
  chain_tensor Lpb = td({8, 1, 4, 256}, BF, kFake + G);
  print_status("merge_dtype", chain_lse_merge(&Ops, &Lpb, &Om, &Lm, nullptr));

  chain_tensor X = td({512, 256}, BF, kFake), W1 = td({256, 128}, BF, kFake + G), W2 = td({128, 256}, BF, kFake + 2 * G),
               Ox = td({512, 256}, BF, kFake + 3 * G);
  const size_t need = chain_mlp_workspace_bytes(512, 128, BF);
  print_status("mlp_workspace_small", chain_mlp_fwd(&X, &W1, &W2, &Ox, 0, (void *)(kFake + 4 * G), need - 1, nullptr));
  print_status("mlp_act", chain_mlp_fwd(&X, &W1, &W2, &Ox, 9, (void *)(kFake + 4 * G), need, nullptr));
  chain_tensor W1b = td({255, 128}, BF, kFake + G);
  print_status("mlp_shape", chain_mlp_fwd(&X, &W1b, &W2, &Ox, 0, (void *)(kFake + 4 * G), need, nullptr));
  print_status("mlp_ws_alias", chain_mlp_fwd(&X, &W1, &W2, &Ox, 0, (void *)(kFake + 256), need, nullptr));
  chain_tensor Xbig = td({8200, 8}, BF, kFake), W1big = td({8, 4096}, BF, kFake + G),
               W2big = td({4096, 8}, BF, kFake + 2 * G), Obig = td({8200, 8}, BF, kFake + 3 * G);
  print_status("mlp_noalloc_beyond_scratch", chain_mlp_fwd_noalloc(&Xbig, &W1big, &W2big, &Obig, 0, nullptr));
  chain_tensor Wg = td({256, 128}, BF, kFake + G, {1, 256}), Wu = td({256, 128}, BF, kFake + 5 * G, {1, 256});
  chain_tensor Wgr = td({256, 128}, BF, kFake + G);
  print_status("gated_rowmajor_gate", chain_mlp_gated_fwd(&X, &Wgr, &Wu, &W2, &Ox, 3, (void *)(kFake + 4 * G), need,
                                                          nullptr));
  print_status("gated_workspace_null", chain_mlp_gated_fwd(&X, &Wg, &Wu, &W2, &Ox, 3, nullptr, need, nullptr));

  chain_tensor dQ = td({1, 4, 256, 64}, F32, kFake + 5 * G), dK = td({1, 2, 256, 64}, F32, kFake + 6 * G),
               dV = td({1, 2, 256, 64}, F32, kFake + 7 * G), dO = td({1, 4, 256, 64}, BF, kFake + 8 * G);
  const size_t bws = chain_attn_bwd_workspace_bytes(1, 4, 256);
  chain_tensor dVal = td({1, 2, 256, 64}, F32, kFake + 6 * G + 256);   // overlaps dK
  print_status("bwd_alias", chain_attn_bwd(&Q, &K, &V, &O, &L, &dO, &dQ, &dK, &dVal, 1, 0.125f,
                                           (void *)(kFake + 9 * G), bws, nullptr));
  print_status("bwd_workspace", chain_attn_bwd(&Q, &K, &V, &O, &L, &dO, &dQ, &dK, &dV, 1, 0.125f,
                                               (void *)(kFake + 9 * G), bws - 256, nullptr));
  chain_tensor Ol = td({1, 4, 256, 64}, F32, kFake + 3 * G), Sin = td({1, 2, 64, 64}, F32, kFake + 5 * G),
               Sbad = td({1, 2, 64, 32}, F32, kFake + 6 * G);
  const size_t lws = chain_linear_attn_workspace_bytes(1, 2, 256, 64);
  print_status("lin_state_shape", chain_linear_attn_fwd(&Q, &K, &V, &Ol, &Sin, &Sbad, (void *)(kFake + 9 * G), lws,
                                                        nullptr));
  print_status("lin_workspace", chain_linear_attn_fwd(&Q, &K, &V, &Ol, &Sin, nullptr, (void *)(kFake + 9 * G),
                                                      lws ? lws - 1 : 0, nullptr));
  int64_t f, d, k;
  print_status("census_null_counts", chain_attn_tile_census(256, nullptr, 256, nullptr, 1, 0, 1, 32, 64, nullptr, &d, &k));
  print_status("census_bad_block", chain_attn_tile_census(256, nullptr, 256, nullptr, 1, 0, 1, 0, 64, &f, &d, &k));
  return 0;
}
