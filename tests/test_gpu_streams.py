"""Calls on caller-chosen streams: the library launches on the stream it is given
(the binding passes torch's current stream) and keeps no state between calls, so
calls interleaved on two streams give the default stream's results bit for bit."""

import pytest
import torch

from gemm_chain_amd import chain
from gemm_chain_amd.workloads import gen_attention, gen_mlp
from gpu_util import announce, device

pytestmark = pytest.mark.gpu


def _kmajor(w):
    return w.t().contiguous().t()


def test_calls_interleaved_on_two_streams_match_the_default_stream():
    dev = device()
    q, k, v = (t.to(dev) for t in gen_attention(1, 8, 2, 1024, 1024, 128, "bf16", 0.5, 31))
    x, w1, w2 = gen_mlp(512, 256, 136, 264, dtype="bf16", amp_x=1.0, amp_w=0.05, seed=32)
    x, w1, w2 = x.to(dev), _kmajor(w1.to(dev)), _kmajor(w2.to(dev))
    announce("streams: default-stream references")
    ref_o, ref_l = chain.attn_fwd(q, k, v, causal=True, n_chunks=2, zigzag=True)
    ref_m = chain.mlp_fwd(x, w1, w2, act="gelu_erf")
    parts = [chain.attn_partial(q, k[:, :, s:s + 512].contiguous(), v[:, :, s:s + 512].contiguous(),
                                [(0, 1024)], [(s, 512)], causal=True) for s in (512, 0)]
    ref_mo, ref_ml = chain.lse_merge(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]))
    torch.cuda.synchronize()

    announce("streams: interleaved on two side streams")
    s1, s2 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)   # default priority
    for s in (s1, s2):
        s.wait_stream(torch.cuda.current_stream(dev))
    stacked = (torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]))
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            o, l = chain.attn_fwd(q, k, v, causal=True, n_chunks=2, zigzag=True)
        with torch.cuda.stream(s2):
            m = chain.mlp_fwd(x, w1, w2, act="gelu_erf")
            mo, ml = chain.lse_merge(*stacked)
        outs.append((o, l, m, mo, ml))
    torch.cuda.synchronize()
    for o, l, m, mo, ml in outs:
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
        assert torch.equal(m, ref_m)
        assert torch.equal(mo, ref_mo) and torch.equal(ml, ref_ml)


def test_results_follow_stream_order():
    """Work queued after a call on the same stream sees its output without a sync."""
    dev = device()
    q, k, v = (t.to(dev) for t in gen_attention(1, 4, 4, 512, 512, 64, "bf16", 0.5, 33))
    announce("streams: ordering on one side stream")
    ref_o, _ = chain.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    s1 = torch.cuda.Stream(device=dev)
    s1.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s1):
        o, _ = chain.attn_fwd(q, k, v, causal=True)
        copy = o.clone()          # queued on s1 after the attention
    torch.cuda.synchronize()
    assert torch.equal(copy, ref_o)
