"""HIP graph capture of library calls: the library only launches kernels on the
caller's stream (no allocation, no memset, no synchronisation), so a captured
sequence of calls replays with the eager results, reading its inputs at replay."""

import pytest
import torch

from gemm_chain_amd import chain
from gemm_chain_amd.workloads import gen_attention, gen_mlp
from gpu_util import announce, device

pytestmark = pytest.mark.gpu


def _kmajor(w):
    return w.t().contiguous().t()


def test_captured_calls_replay_the_eager_results():
    dev = device()
    q, k, v = (t.to(dev) for t in gen_attention(1, 8, 2, 1024, 1024, 128, "bf16", 0.5, 41))
    x, w1, w2 = gen_mlp(512, 256, 136, 264, dtype="bf16", amp_x=1.0, amp_w=0.05, seed=42)
    x, w1, w2 = x.to(dev), _kmajor(w1.to(dev)), _kmajor(w2.to(dev))
    o = torch.empty_like(q)
    l = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    m = torch.empty((x.shape[0], w2.shape[1]), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(chain.mlp_workspace_bytes(x.shape[0], w1.shape[1]), dtype=torch.uint8, device=dev)
    po = torch.empty((2,) + tuple(q.shape), dtype=torch.float32, device=dev)
    pl = torch.empty((2,) + tuple(q.shape[:3]), dtype=torch.float32, device=dev)
    mo = torch.empty_like(q)
    ml = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def calls():
        chain.attn_fwd(q, k, v, causal=True, n_chunks=2, zigzag=True, out=o, lse=l)
        chain.mlp_fwd(x, w1, w2, act="gelu_erf", out=m, workspace=ws)
        for i, s in enumerate((512, 0)):
            chain.attn_partial(q, k[:, :, s:s + 512], v[:, :, s:s + 512], [(0, 1024)], [(s, 512)],
                               causal=True, out=po[i], lse=pl[i])
        chain.lse_merge(po, pl, out=mo, lse=ml)

    def eager():
        calls()
        torch.cuda.synchronize()
        return [t.clone() for t in (o, l, m, mo, ml)]

    announce("graphs: warm-up and capture")
    ref = eager()                      # warm-up outside the capture (first-call setup)
    s = torch.cuda.Stream(device=dev)  # default priority
    s.wait_stream(torch.cuda.current_stream(dev))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    torch.cuda.synchronize()

    gen = torch.Generator(device="cpu").manual_seed(43)
    for rep in range(3):
        announce(f"graphs: replay {rep}")
        if rep > 0:   # new input values, written in place between replays
            q.copy_((torch.randn(q.shape, generator=gen) * 0.5).to(torch.bfloat16))
            x.copy_(torch.randn(x.shape, generator=gen).to(torch.bfloat16))
            ref = eager()
        for t in (o, l, m, mo, ml):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((o, l, m, mo, ml), ref):
            assert torch.equal(got, want), rep
