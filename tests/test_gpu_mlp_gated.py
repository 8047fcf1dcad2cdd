"""GPU parity of chain_mlp_gated_fwd (O = (act(X.Wg) * (X.Wu)).Wd) against the
float64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from gemm_chain_amd import chain
from gemm_chain_amd.workloads import WORKLOADS, gen_mlp_gated
from gpu_util import TOL_BF16, announce, device, f64, max_abs, sample_rows

pytestmark = pytest.mark.gpu


def _kmajor(w):
    """The same [K, N] values stored column-major (a row-major [N, K] array, transposed)."""
    return w.t().contiguous().t()


# Weights drawn at N(0, amp^2) so that the outputs stay in the workload's
# magnitude range; the bound is absolute (bf16 inputs, f32 accumulation).
@pytest.mark.parametrize("M,K,N,K2,act,out", [
    (300, 256, 136, 264, "silu", None),        # ragged M, N and K2 tiles
    (300, 256, 136, 264, "gelu_erf", None),
    (300, 256, 136, 264, "identity", "f32"),   # f32 output: no output rounding
    (257, 4096, 1376, 512, "silu", None),      # gated FFN shard inner width, full K
    (64, 64, 8, 64, "silu", "f32"),            # a single 8-column inner block
    (300, 136, 264, 200, "silu", None),        # K tail in the gate/up product, N and K2 ragged
])
def test_gated_mlp_small_full_compare(M, K, N, K2, act, out):
    dev = device()
    x, wg, wu, wd = gen_mlp_gated(M, K, N, K2, amp_x=1.0, amp_w=0.02 if K > 512 else 0.05, seed=80 + M + N)
    announce(f"mlp_gated M{M} K{K} N{N} K2{K2} {act} out {out}")
    o = chain.mlp_gated_fwd(x.to(dev), _kmajor(wg.to(dev)), _kmajor(wu.to(dev)), wd.to(dev), act=act,
                            out_dtype=torch.float32 if out == "f32" else None)
    torch.cuda.synchronize()
    ref = oracle.mlp_gated(f64(x), f64(wg), f64(wu), f64(wd), act)
    err = max_abs(f64(o), ref)
    print(f"max-abs {err:.3e}  max|ref| {np.abs(ref).max():.3e}")
    assert err <= TOL_BF16


def test_gated_mlp_ffn_shard_m16384_sampled():
    w = WORKLOADS["mlp_gated_bf16_m16384_k4096_n1376"]
    dev = device()
    x, wg, wu, wd = gen_mlp_gated(w.M, w.K, w.N, dtype=w.dtype, amp_x=w.amp_x, amp_w=w.amp_w, seed=w.seed)
    announce("mlp_gated 16384x4096x1376 full size")
    o = chain.mlp_gated_fwd(x.to(dev), _kmajor(wg.to(dev)), _kmajor(wu.to(dev)), _kmajor(wd.to(dev)),
                            act=w.act)
    torch.cuda.synchronize()
    rows = sample_rows(w.M, 160, w.seed, extra=(127, 128, 255, 256, 8191))
    ref = oracle.mlp_gated(f64(x[rows]), f64(wg), f64(wu), f64(wd), w.act)
    err = max_abs(f64(o.cpu()[rows]), ref)
    print(f"max-abs {err:.3e} over {len(rows)} rows")
    assert err <= TOL_BF16


def test_gated_mlp_row_stride_beyond_32bit_tile_offsets():
    """X rows 4.4 M elements apart: a 256-row tile of X spans more than 2^31 bytes, so the
    gate/up product runs on the four-wave kernel (64-bit addresses) and H.Wd on the
    eight-wave one; the result equals the contiguous call's bit for bit."""
    dev = device()
    M, K, N, K2, lda = 300, 128, 136, 96, 4_400_000
    x, wg, wu, wd = gen_mlp_gated(M, K, N, K2, amp_x=1.0, amp_w=0.05, seed=86)
    xd = x.to(dev)
    wgd, wud, wdd = _kmajor(wg.to(dev)), _kmajor(wu.to(dev)), _kmajor(wd.to(dev))
    announce(f"mlp_gated X row stride {lda} (tile span beyond 2^31 bytes)")
    store = torch.zeros((M - 1) * lda + K, dtype=torch.bfloat16, device=dev)
    xs = store.as_strided((M, K), (lda, 1))
    xs.copy_(xd)
    o = chain.mlp_gated_fwd(xs, wgd, wud, wdd, act="silu")
    dense = chain.mlp_gated_fwd(xd, wgd, wud, wdd, act="silu")
    torch.cuda.synchronize()
    assert torch.equal(o, dense)
    ref = oracle.mlp_gated(f64(x), f64(wg), f64(wu), f64(wd), "silu")
    assert max_abs(f64(o), ref) <= TOL_BF16
    del store, xs


def test_gated_mlp_down_weight_layouts_agree():
    """Wd row- or column-major: the same products in the same k order."""
    dev = device()
    x, wg, wu, wd = gen_mlp_gated(1000, 512, 392, 264, amp_x=1.0, amp_w=0.05, seed=90)
    xd, wgd, wud, wdd = x.to(dev), _kmajor(wg.to(dev)), _kmajor(wu.to(dev)), wd.to(dev)
    announce("mlp_gated down-weight layouts")
    a = chain.mlp_gated_fwd(xd, wgd, wud, wdd)
    b = chain.mlp_gated_fwd(xd, wgd, wud, _kmajor(wdd))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _gated_width(M, N, cus=256):
    """The library's gated tile choice: 32 x nbw output columns, nbw 2 unless 4
    takes no more rounds x nbw."""
    def cost(nbw):
        tiles = -(-M // 256) * -(-N // (32 * nbw))
        return -(-tiles // cus) * nbw
    return 2 if cost(2) < cost(4) else 4


@pytest.mark.parametrize("M,K,N,K2,pad,nbw", [
    (300, 256, 136, 264, 0, 2),      # last inner tile of 8 columns
    (4096, 1376, 4096, 264, 0, 4),   # 128-wide tiles, whole stages
    (4000, 264, 4000, 136, 0, 4),    # 128-wide tiles, ragged N, a K tail after eight stages
    (96, 24, 40, 16, 0, 2),          # K inside one partial stage
    (4096, 24, 4096, 264, 0, 4),     # 128-wide tiles (64-deep stages) with K inside one partial stage
    (1000, 512, 392, 264, 24, 2),    # gate and up rows padded past N
    (16384, 4096, 1376, 4096, 0, 4),  # the FFN shard
])
def test_gated_mlp_gate_up_layouts_agree(M, K, N, K2, pad, nbw):
    """Row-major gate and up weights give the bits of column-major ones (the same
    products in the same k order), and match the oracle on sampled rows."""
    dev = device()
    if torch.cuda.get_device_properties(dev).multi_processor_count != 256:
        pytest.skip("the tile choice asserted here assumes 256 compute units")
    assert _gated_width(M, N) == nbw
    x, wg, wu, wd = gen_mlp_gated(M, K, N, K2, amp_x=1.0, amp_w=0.02 if K > 512 else 0.05, seed=95 + M % 89)
    announce(f"mlp_gated gate/up layouts M{M} K{K} N{N} K2{K2} pad {pad}")
    xd, wdd = x.to(dev), wd.to(dev)

    def rowmajor(w):
        buf = torch.zeros(K, N + pad, dtype=w.dtype, device=dev)
        buf[:, :N] = w.to(dev)
        return buf[:, :N]
    o_r = chain.mlp_gated_fwd(xd, rowmajor(wg), rowmajor(wu), wdd, act="silu")
    o_k = chain.mlp_gated_fwd(xd, _kmajor(wg.to(dev)), _kmajor(wu.to(dev)), wdd, act="silu")
    torch.cuda.synchronize()
    assert torch.equal(o_r, o_k)
    rows = sample_rows(M, 48, 95, extra=(0, M - 1, min(M - 1, 255), min(M - 1, 256)))
    ref = oracle.mlp_gated(f64(x[rows]), f64(wg), f64(wu), f64(wd), "silu")
    err = max_abs(f64(o_r.cpu()[rows]), ref)
    print(f"max-abs {err:.3e} over {len(rows)} rows")
    assert err <= TOL_BF16


def test_gated_mlp_shard_sum_equals_whole():
    """Inner-dimension shards of gate, up and down summed give the unsharded chain
    (f32 output: the bf16 intermediate is rounded element by element either way)."""
    dev = device()
    x, wg, wu, wd = gen_mlp_gated(256, 256, 512, 256, amp_x=1.0, amp_w=0.05, seed=91)
    xd, wgd, wud, wdd = x.to(dev), wg.to(dev), wu.to(dev), wd.to(dev)
    announce("mlp_gated shard sum")
    whole = chain.mlp_gated_fwd(xd, _kmajor(wgd), _kmajor(wud), wdd, out_dtype=torch.float32)
    parts = sum(chain.mlp_gated_fwd(xd, _kmajor(wgd[:, s:s + 128]), _kmajor(wud[:, s:s + 128]),
                                    wdd[s:s + 128].contiguous(), out_dtype=torch.float32)
                for s in range(0, 512, 128))
    torch.cuda.synchronize()
    assert (whole - parts).abs().max().item() <= 1e-4


def test_gated_mlp_zero_input_and_empty_inner():
    dev = device()
    _, wg, wu, wd = gen_mlp_gated(8, 64, 64, 64, seed=92)
    announce("mlp_gated X = 0, N = 0")
    x = torch.zeros(128, 64, dtype=torch.bfloat16, device=dev)
    o = chain.mlp_gated_fwd(x, _kmajor(wg.to(dev)), _kmajor(wu.to(dev)), wd.to(dev))
    e = torch.full((128, 64), 3.0, dtype=torch.bfloat16, device=dev)
    chain.mlp_gated_fwd(x + 1, torch.empty(64, 0, dtype=torch.bfloat16, device=dev).t().t(),
                        torch.empty(64, 0, dtype=torch.bfloat16, device=dev), torch.empty(0, 64, dtype=torch.bfloat16, device=dev),
                        out=e)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(e == 0)
