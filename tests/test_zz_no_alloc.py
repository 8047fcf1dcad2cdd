"""chain_mlp_fwd_noalloc: the MLP chain with its intermediate in the library's
static per-GPU scratch gives the bits of chain_mlp_fwd with a caller workspace,
call after call, and refuses shapes whose intermediate does not fit."""

import numpy as np
import pytest
import torch

import oracle
from gemm_chain_amd import chain
from gemm_chain_amd.workloads import gen_mlp
from gpu_util import TOL_BF16, announce, device, f64, max_abs

pytestmark = pytest.mark.gpu

# (M, K, N, K2, act, column-major weights): the second case is smaller than the
# first, so the scratch still holds the first call's larger intermediate.
CASES = [(1000, 512, 1376, 512, "gelu_erf", True), (200, 256, 136, 256, "silu", False)]


def _weights(w, colmajor):
    return w.t().contiguous().t() if colmajor else w


def test_noalloc_matches_workspace_call_twice():
    dev = device()
    for i, (M, K, N, K2, act, colmajor) in enumerate(CASES):
        x, w1, w2 = gen_mlp(M, K, N, K2, dtype="bf16", amp_x=1.0, amp_w=0.02, seed=40 + i)
        xd = x.to(dev)
        w1d, w2d = _weights(w1.to(dev), colmajor), _weights(w2.to(dev), colmajor)
        announce(f"noalloc mlp call {i}: M{M} K{K} N{N} K2{K2} {act}")
        got = chain.mlp_fwd_noalloc(xd, w1d, w2d, act=act)
        ref = chain.mlp_fwd(xd, w1d, w2d, act=act)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"call {i}: bits differ from chain_mlp_fwd"
        err = max_abs(f64(got), oracle.mlp(f64(x), f64(w1), f64(w2), act))
        print(f"call {i}: max-abs vs oracle {err:.3e}")
        assert err <= TOL_BF16


def test_noalloc_refuses_intermediate_beyond_scratch():
    dev = device()
    # H = 8200 x 4096 bf16 = 67,174,400 bytes > 64 MiB; everything else is tiny.
    M, K, N = 8200, 8, 4096
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    w1 = torch.zeros((K, N), dtype=torch.bfloat16, device=dev)
    w2 = torch.zeros((N, K), dtype=torch.bfloat16, device=dev)
    o = torch.full((M, K), 7.0, dtype=torch.bfloat16, device=dev)
    announce("noalloc mlp beyond the scratch")
    with pytest.raises(chain.ChainError) as e:
        chain.mlp_fwd_noalloc(x, w1, w2, out=o)
    assert e.value.name == "CHAIN_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)          # refused before anything ran
    # one row fewer in N fits: 8200 x 4088 x 2 = 67,043,200 bytes
    w1s, w2s = w1[:, :4088].contiguous(), w2[:4088].contiguous()
    got = chain.mlp_fwd_noalloc(x, w1s, w2s, out=o)
    torch.cuda.synchronize()
    assert torch.all(got == 0)
