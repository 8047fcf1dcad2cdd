"""GPU parity of chain_mlp_fwd (O = act(X.W1).W2) against the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from gemm_chain_amd import chain
from gemm_chain_amd.workloads import WORKLOADS, gen_mlp
from gpu_util import TOL_BF16, TOL_F32, announce, device, f64, max_abs, sample_rows

pytestmark = pytest.mark.gpu


# Weights drawn like the FFN shard workload (N(0, 0.02^2)) so that outputs stay
# in the same magnitude range; the bound is absolute, and a bf16 output of
# magnitude 4..8 alone carries up to 1.6e-2 of rounding.
@pytest.mark.parametrize("M,K,N,K2,dtype,act,out", [
    (300, 256, 136, 264, "bf16", "gelu_erf", None),       # ragged M, N and K2 tiles
    (257, 4096, 1376, 512, "bf16", "gelu_tanh", None),    # FFN shard inner width, full K
    (257, 4096, 1376, 512, "bf16", "gelu_erf", "f32"),    # f32 output: no output rounding
    (64, 128, 64, 128, "bf16", "identity", None),
    (200, 136, 72, 96, "f32", "gelu_erf", None),          # f32 MFMA path
])
def test_mlp_small_full_compare(M, K, N, K2, dtype, act, out):
    dev = device()
    x, w1, w2 = gen_mlp(M, K, N, K2, dtype=dtype, amp_x=1.0, amp_w=0.02 if K > 512 else 0.05,
                        seed=40 + M)
    announce(f"mlp M{M} K{K} N{N} K2{K2} {dtype} {act} out {out}")
    o = chain.mlp_fwd(x.to(dev), w1.to(dev), w2.to(dev), act=act,
                      out_dtype=torch.float32 if out == "f32" else None)
    torch.cuda.synchronize()
    ref = oracle.mlp(f64(x), f64(w1), f64(w2), act)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    err = max_abs(f64(o), ref)
    print(f"max-abs {err:.3e}")
    assert err <= tol


@pytest.mark.parametrize("kmajor", [False, True])
def test_mlp_ffn_shard_m16384_sampled(kmajor):
    """Full size, with the weights row-major or (as the bench times them) k-major."""
    w = WORKLOADS["mlp_bf16_m16384_k4096_n1376"]
    dev = device()
    x, w1, w2 = gen_mlp(w.M, w.K, w.N, dtype=w.dtype, amp_x=w.amp_x, amp_w=w.amp_w, seed=w.seed)
    announce(f"mlp 16384x4096x1376 full size kmajor={kmajor}")
    w1d, w2d = w1.to(dev), w2.to(dev)
    if kmajor:
        w1d, w2d = _kmajor(w1d), _kmajor(w2d)
    o = chain.mlp_fwd(x.to(dev), w1d, w2d, act=w.act)
    torch.cuda.synchronize()
    rows = sample_rows(w.M, 160, w.seed, extra=(127, 128, 8191))
    ref = oracle.mlp(f64(x[rows]), f64(w1), f64(w2), w.act)
    err = max_abs(f64(o.cpu()[rows]), ref)
    print(f"max-abs {err:.3e} over {len(rows)} rows")
    assert err <= TOL_BF16


def _rounds_x_width(M, N, width, cus=256):
    """The library's tile-width cost: rounds x (width + 64)."""
    tiles = -(-M // 256) * -(-N // width)
    return -(-tiles // cus) * (width + 64)


def test_mlp_wide_tiles_ragged():
    """An X.W1 whose inner width takes the 352-wide uneven tiles on a 256-CU chip
    (one round, where 128-, 192- and 256-wide tiles need two or three), with a
    ragged last row tile, a ragged last column tile and a K tail; k-major and
    row-major weights both take those tiles (B staged per column or per k row)
    and must give the same bits."""
    M, K, N, K2 = 8092, 4104, 2792, 512
    assert _rounds_x_width(M, N, 352) < min(_rounds_x_width(M, N, w) for w in (128, 192, 256))
    dev = device()
    if torch.cuda.get_device_properties(dev).multi_processor_count != 256:
        pytest.skip("the tile choice asserted here assumes 256 compute units")
    x, w1, w2 = gen_mlp(M, K, N, K2, dtype="bf16", amp_x=1.0, amp_w=0.02, seed=53)
    announce(f"mlp wide tiles M{M} K{K} N{N} K2{K2}")
    xd, w1d, w2d = x.to(dev), w1.to(dev), w2.to(dev)
    o_row = chain.mlp_fwd(xd, w1d, w2d, act="gelu_erf")
    o_k = chain.mlp_fwd(xd, _kmajor(w1d), _kmajor(w2d), act="gelu_erf")
    torch.cuda.synchronize()
    assert torch.equal(o_row, o_k)
    rows = sample_rows(M, 120, 53, extra=(0, 255, 256, 7935, 7936, M - 1))
    ref = oracle.mlp(f64(x[rows]), f64(w1), f64(w2), "gelu_erf")
    err = max_abs(f64(o_k.cpu()[rows]), ref)
    print(f"max-abs {err:.3e} over {len(rows)} rows")
    assert err <= TOL_BF16


@pytest.mark.parametrize("K,pad", [(24, 0), (4104, 40), (64, 8)])
def test_mlp_row_major_wide_tiles_edges(K, pad):
    """Row-major weights on the 352-wide tiles: a last column tile of 8 columns
    (N = 7 x 352 + 8), K within one partial stage (24), a K tail after whole
    stages (4104) and whole stages only (64), W1 rows padded past N (a view of
    a wider array); the bits must equal those of k-major weights."""
    M, N, K2 = 8092, 7 * 352 + 8, 264
    assert _rounds_x_width(M, N, 352) < min(_rounds_x_width(M, N, w) for w in (128, 192, 256))
    dev = device()
    if torch.cuda.get_device_properties(dev).multi_processor_count != 256:
        pytest.skip("the tile choice asserted here assumes 256 compute units")
    x, w1, w2 = gen_mlp(M, K, N, K2, dtype="bf16", amp_x=1.0, amp_w=0.02, seed=70 + K % 89)
    announce(f"mlp row-major wide tiles M{M} K{K} N{N} K2{K2} pad {pad}")
    xd, w2d = x.to(dev), w2.to(dev)
    w1p = torch.zeros(K, N + pad, dtype=w1.dtype, device=dev)
    w1p[:, :N] = w1.to(dev)
    w1d = w1p[:, :N]
    o_row = chain.mlp_fwd(xd, w1d, w2d, act="gelu_tanh")
    o_k = chain.mlp_fwd(xd, _kmajor(w1d), _kmajor(w2d), act="gelu_tanh")
    torch.cuda.synchronize()
    assert torch.equal(o_row, o_k)
    rows = sample_rows(M, 64, 70, extra=(0, 255, 256, 7935, 7936, M - 1))
    ref = oracle.mlp(f64(x[rows]), f64(w1), f64(w2), "gelu_tanh")
    err = max_abs(f64(o_row.cpu()[rows]), ref)
    print(f"max-abs {err:.3e} over {len(rows)} rows")
    assert err <= TOL_BF16


def test_mlp_shard_sum_equals_whole():
    """Summing the outputs of inner-dimension shards gives the unsharded chain."""
    dev = device()
    x, w1, w2 = gen_mlp(256, 256, 512, 256, dtype="f32", amp_x=1.0, amp_w=0.05, seed=50)
    xd, w1d, w2d = x.to(dev), w1.to(dev), w2.to(dev)
    announce("mlp shard sum")
    whole = chain.mlp_fwd(xd, w1d, w2d, act="gelu_erf")
    parts = sum(chain.mlp_fwd(xd, w1d[:, s:s + 128].contiguous(), w2d[s:s + 128].contiguous(),
                              act="gelu_erf") for s in range(0, 512, 128))
    assert (whole - parts).abs().max().item() <= 1e-4


def test_mlp_zero_input():
    dev = device()
    _, w1, w2 = gen_mlp(8, 64, 64, 64, seed=51)
    x = torch.zeros(128, 64, dtype=torch.bfloat16, device=dev)
    announce("mlp X = 0")
    o = chain.mlp_fwd(x, w1.to(dev), w2.to(dev))
    assert torch.all(o == 0)


def _kmajor(w):
    """The same [K, N] values stored column-major (a row-major [N, K] array, transposed)."""
    return w.t().contiguous().t()


# On a 256-CU device these shapes select each bf16 tile width: 256- and
# 352-wide tiles take 64-deep stages, narrower ones 32-deep.  M, N or K is
# ragged in each.
@pytest.mark.parametrize("M,K,N,K2", [
    (16000, 4096, 1376, 4096),  # 352 and 352 wide; H.W2 with a K tail (1376 = 21 x 64 + 32)
    (4000, 1376, 4096, 264),    # 256 wide with a K tail, then 128 wide
    (4000, 4096, 4096, 264),    # 256 wide, whole 64-deep stages, then 128 wide
    (12000, 4032, 1376, 256),   # 352 wide over 63 whole stages, then 128 wide
    (17900, 72, 1152, 264),     # 192 wide (uneven loads of B per wave), a K tail after two stages
    (300, 200, 136, 264),       # 128 wide
    (96, 8, 24, 40),            # K and N below one 32-deep stage: only K-tail stages
    (16000, 4008, 1376, 264),   # 352 wide with a K tail (4008 = 62 x 64 + 40)
    (33, 40, 8, 16),            # one partial row tile, one 8-column inner block
])
def test_mlp_weight_layouts_agree_and_match_oracle(M, K, N, K2):
    dev = device()
    x, w1, w2 = gen_mlp(M, K, N, K2, dtype="bf16", amp_x=1.0, amp_w=0.02, seed=60 + M % 97)
    xd, w1d, w2d = x.to(dev), w1.to(dev), w2.to(dev)
    announce(f"mlp layouts M{M} K{K} N{N} K2{K2}")
    o_row = chain.mlp_fwd(xd, w1d, w2d, act="gelu_erf")
    o_col = chain.mlp_fwd(xd, _kmajor(w1d), _kmajor(w2d), act="gelu_erf")
    o_mix = chain.mlp_fwd(xd, _kmajor(w1d), w2d, act="gelu_erf")
    torch.cuda.synchronize()
    # Same products in the same k order whatever the weight layout.
    assert torch.equal(o_row, o_col) and torch.equal(o_row, o_mix)
    rows = sample_rows(M, 96, 7, extra=(0, M - 1, min(M - 1, 255), min(M - 1, 256)))
    ref = oracle.mlp(f64(x[rows]), f64(w1), f64(w2), "gelu_erf")
    err = max_abs(f64(o_col.cpu()[rows]), ref)
    print(f"max-abs {err:.3e} over {len(rows)} rows")
    assert err <= TOL_BF16


def test_mlp_row_stride_beyond_32bit_tile_offsets():
    """X rows 4.4 M elements apart: a 256-row tile of X spans more than 2^31 bytes, so
    X.W1 runs on the four-wave kernel (64-bit addresses) while H.W2 runs on the
    eight-wave kernel; both use the same k order, so the result equals the contiguous
    call's bit for bit."""
    dev = device()
    M, K, N, K2, lda = 300, 128, 136, 96, 4_400_000
    x, w1, w2 = gen_mlp(M, K, N, K2, dtype="bf16", amp_x=1.0, amp_w=0.05, seed=75)
    xd, w1d, w2d = x.to(dev), _kmajor(w1.to(dev)), _kmajor(w2.to(dev))
    announce(f"mlp X row stride {lda} (tile span beyond 2^31 bytes)")
    store = torch.zeros((M - 1) * lda + K, dtype=torch.bfloat16, device=dev)
    xs = store.as_strided((M, K), (lda, 1))
    xs.copy_(xd)
    o = chain.mlp_fwd(xs, w1d, w2d, act="gelu_erf")
    dense = chain.mlp_fwd(xd, w1d, w2d, act="gelu_erf")
    torch.cuda.synchronize()
    assert torch.equal(o, dense)
    ref = oracle.mlp(f64(x), f64(w1), f64(w2), "gelu_erf")
    assert max_abs(f64(o), ref) <= TOL_BF16
    del store, xs


def test_mlp_row_major_weight_stride_beyond_32bit_offsets():
    """Row-major W2 rows 20 M elements apart: its column band spans more than 2^31
    bytes, so H.W2 runs on the register-staged kernel (64-bit addresses) instead of
    the direct-to-LDS one; the same k order gives the contiguous call's bits."""
    dev = device()
    M, K, N, K2, ldb = 300, 128, 136, 96, 20_000_000
    x, w1, w2 = gen_mlp(M, K, N, K2, dtype="bf16", amp_x=1.0, amp_w=0.05, seed=76)
    xd, w1d, w2d = x.to(dev), w1.to(dev), w2.to(dev)
    announce(f"mlp row-major W2 row stride {ldb} (band beyond 2^31 bytes)")
    store = torch.zeros((N - 1) * ldb + K2, dtype=torch.bfloat16, device=dev)
    w2s = store.as_strided((N, K2), (ldb, 1))
    w2s.copy_(w2d)
    o = chain.mlp_fwd(xd, w1d, w2s, act="gelu_erf")
    dense = chain.mlp_fwd(xd, w1d, w2d, act="gelu_erf")
    torch.cuda.synchronize()
    assert torch.equal(o, dense)
    ref = oracle.mlp(f64(x), f64(w1), f64(w2), "gelu_erf")
    assert max_abs(f64(o), ref) <= TOL_BF16
    del store, w2s


@pytest.mark.parametrize("w2_kmajor", [False, True])
@pytest.mark.parametrize("pad", [2, 4])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_mlp_output_row_stride_not_vector_aligned(out_dtype, pad, w2_kmajor):
    """An output whose row stride is not a multiple of 4 elements (pad 2: element stores)
    or, in bf16, of 8 elements (pad 4: 8-byte stores instead of 16-byte ones), written by
    the row-major-weight kernel or (W2 k-major) the eight-wave kernel."""
    dev = device()
    M, K, N, K2 = 260, 128, 136, 200
    x, w1, w2 = gen_mlp(M, K, N, K2, dtype="bf16", amp_x=1.0, amp_w=0.05, seed=70)
    xd, w1d, w2d = x.to(dev), _kmajor(w1.to(dev)), w2.to(dev)
    if w2_kmajor:
        w2d = _kmajor(w2d)
    announce(f"mlp strided output {out_dtype} pad {pad} w2_kmajor {w2_kmajor}")
    base = torch.full((M, K2 + pad), 7.0, dtype=out_dtype, device=dev)
    o = base[:, :K2]
    chain.mlp_fwd(xd, w1d, w2d, act="gelu_tanh", out=o)
    dense = chain.mlp_fwd(xd, w1d, w2d, act="gelu_tanh", out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(o, dense)
    assert torch.all(base[:, K2:] == 7.0)
    ref = oracle.mlp(f64(x), f64(w1), f64(w2), "gelu_tanh")
    assert max_abs(f64(o), ref) <= TOL_BF16


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kmajor", [False, True])
def test_mlp_empty_inner_dimensions(dtype, kmajor):
    """K = 0 gives H = act(0) = 0 and N = 0 an empty intermediate: O = 0 either way."""
    dev = device()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    M, K2 = 300, 264
    announce(f"mlp empty inner dims {dtype} kmajor={kmajor}")
    for K, N in ((0, 136), (128, 0)):
        x = torch.randn(M, K, device=dev).to(tdt)
        w1 = torch.randn(K, N, device=dev).to(tdt)
        w2 = torch.randn(N, K2, device=dev).to(tdt)
        if kmajor:
            w1, w2 = _kmajor(w1), _kmajor(w2)
        o = torch.full((M, K2), 5.0, dtype=tdt, device=dev)
        chain.mlp_fwd(x, w1, w2, act="gelu_erf", out=o)
        torch.cuda.synchronize()
        assert torch.all(o == 0), (K, N)


@pytest.mark.parametrize("act", ["gelu_erf", "gelu_tanh", "silu"])
def test_mlp_activation_accuracy_f32(act):
    """X.I.I in f32 isolates the activation: O = act(X) up to its approximation error
    (the erf form uses a rational approximation with |error| <= 1.5e-7; SiLU uses the
    hardware exp2 and reciprocal, about one ulp each)."""
    dev = device()
    M, N = 512, 64
    z = torch.linspace(-9.0, 9.0, M * N, dtype=torch.float64).reshape(M, N)
    x = z.to(torch.float32)
    eye = torch.eye(N, dtype=torch.float32)
    announce(f"mlp activation accuracy {act}")
    o = chain.mlp_fwd(x.to(dev), eye.to(dev), eye.to(dev), act=act)
    torch.cuda.synchronize()
    ref = oracle.ACTIVATIONS[act](f64(x))
    err = np.abs(f64(o) - ref)
    bound = 1e-6 + 2e-7 * np.abs(f64(x))
    print(f"max-abs {err.max():.3e}")
    assert np.all(err <= bound)
