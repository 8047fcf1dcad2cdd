"""Seeded synthetic inputs for the chain workloads.

This module holds no arithmetic of the method: it only draws random tensors of
the shapes and distributions of the workloads, so that the HIP path (through
the binding) and the float64 oracle receive bit-identical inputs.  Recipe for
every tensor: a torch CPU ``Generator`` seeded with the workload's seed draws
``randn`` in float32, in the order the tensors are listed, each scaled by its
amplitude and then cast to the workload's dtype (float32 -> bfloat16 rounds to
nearest even).  The oracle receives the same values widened to float64.

Shapes follow the 7B dense decoder the TSP article measures (hidden size 4096,
32 heads, so head_dim 128) and the GQA grouping of the 2D-Attention summary.
"""

import math
from dataclasses import dataclass, field

import torch

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class AttnWorkload:
    name: str
    dtype: str            # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    S: int                # keys (and queries unless a share is taken)
    D: int
    amp: float
    seed: int
    n_chunks: int = 1
    zigzag: bool = False
    ring_ranks: int = 0   # >0: one rank's zigzag share of the queries
    ring_rank: int = 0

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)


@dataclass(frozen=True)
class MlpWorkload:
    name: str
    dtype: str
    M: int
    K: int
    N: int
    amp_x: float
    amp_w: float
    seed: int
    act: str = "gelu_erf"
    gated: bool = False   # (act(X.Wg) * (X.Wu)).Wd with Wg, Wu [K, N] and Wd [N, K]


WORKLOADS = {
    # single-head causal fp32 attention, one KV chunk
    "attn_f32_s256_d64": AttnWorkload("attn_f32_s256_d64", "f32", 1, 1, 1, 256, 64, 1.0, 1),
    # multi-head causal bf16 attention, single pass, O plus LSE
    "attn_bf16_b2_h32_s4096_d128": AttnWorkload(
        "attn_bf16_b2_h32_s4096_d128", "bf16", 2, 32, 32, 4096, 128, 0.5, 2),
    # rank 0 of an 8-rank zigzag ring over a 32768-token causal context,
    # 8 zigzag KV chunks of 4096 merged by log-sum-exp
    "ring_share_bf16_h32_s32768_r0of8": AttnWorkload(
        "ring_share_bf16_h32_s32768_r0of8", "bf16", 1, 32, 32, 32768, 128, 1.0, 3,
        n_chunks=8, zigzag=True, ring_ranks=8, ring_rank=0),
    # one 8-way shard of an 11008-wide FFN: GeLU(X.W1).W2
    "mlp_bf16_m16384_k4096_n1376": MlpWorkload(
        "mlp_bf16_m16384_k4096_n1376", "bf16", 16384, 4096, 1376, 1.0, 0.02, 4),
    # one 8-way shard of an 11008-wide gated FFN: (SiLU(X.Wg) * (X.Wu)).Wd
    "mlp_gated_bf16_m16384_k4096_n1376": MlpWorkload(
        "mlp_gated_bf16_m16384_k4096_n1376", "bf16", 16384, 4096, 1376, 1.0, 0.02, 6, act="silu",
        gated=True),
    # one device's share (32768 tokens, e.g. 4096K tokens over 128 devices) of causal
    # linear attention with a carried key/value state, 32 heads of 128
    "lin_attn_bf16_h32_s32768_d128": AttnWorkload(
        "lin_attn_bf16_h32_s32768_d128", "bf16", 1, 32, 32, 32768, 128, 0.25, 7),
    # long causal GQA attention, 32 query heads over 8 KV heads, 16 zigzag chunks
    "attn_gqa_bf16_h32kv8_s65536_d128": AttnWorkload(
        "attn_gqa_bf16_h32kv8_s65536_d128", "bf16", 1, 32, 8, 65536, 128, 1.0, 5,
        n_chunks=16, zigzag=True),
}


def gen_attention(B, Hq, Hkv, Sq, Sk, D, dtype="bf16", amp=1.0, seed=0):
    """Q [B,Hq,Sq,D], K and V [B,Hkv,Sk,D] on the CPU, drawn in the order Q, K, V."""
    g = torch.Generator().manual_seed(seed)
    dt = _DTYPES[dtype]
    q = (torch.randn(B, Hq, Sq, D, generator=g, dtype=torch.float32) * amp).to(dt)
    k = (torch.randn(B, Hkv, Sk, D, generator=g, dtype=torch.float32) * amp).to(dt)
    v = (torch.randn(B, Hkv, Sk, D, generator=g, dtype=torch.float32) * amp).to(dt)
    return q, k, v


def gen_attention_grad(B, Hq, S, D, dtype="bf16", amp=1.0, seed=0):
    """dO [B,Hq,S,D] on the CPU: the output gradient fed to the attention backward."""
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(B, Hq, S, D, generator=g, dtype=torch.float32) * amp).to(_DTYPES[dtype])


def gen_linear_state(B, Hkv, D, amp=1.0, seed=0):
    """A carried key/value state S_in [B,Hkv,D,D] in f32 on the CPU (N(0, amp^2))."""
    g = torch.Generator().manual_seed(seed)
    return torch.randn(B, Hkv, D, D, generator=g, dtype=torch.float32) * amp


def gen_mlp(M, K, N, K2=None, dtype="bf16", amp_x=1.0, amp_w=0.02, seed=0):
    """X [M,K], W1 [K,N], W2 [N,K2] on the CPU, drawn in the order X, W1, W2."""
    K2 = K if K2 is None else K2
    g = torch.Generator().manual_seed(seed)
    dt = _DTYPES[dtype]
    x = (torch.randn(M, K, generator=g, dtype=torch.float32) * amp_x).to(dt)
    w1 = (torch.randn(K, N, generator=g, dtype=torch.float32) * amp_w).to(dt)
    w2 = (torch.randn(N, K2, generator=g, dtype=torch.float32) * amp_w).to(dt)
    return x, w1, w2


def gen_mlp_gated(M, K, N, K2=None, dtype="bf16", amp_x=1.0, amp_w=0.02, seed=0):
    """X [M,K], Wg and Wu [K,N], Wd [N,K2] on the CPU, drawn in the order X, Wg, Wu, Wd."""
    K2 = K if K2 is None else K2
    g = torch.Generator().manual_seed(seed)
    dt = _DTYPES[dtype]
    x = (torch.randn(M, K, generator=g, dtype=torch.float32) * amp_x).to(dt)
    wg = (torch.randn(K, N, generator=g, dtype=torch.float32) * amp_w).to(dt)
    wu = (torch.randn(K, N, generator=g, dtype=torch.float32) * amp_w).to(dt)
    wd = (torch.randn(N, K2, generator=g, dtype=torch.float32) * amp_w).to(dt)
    return x, wg, wu, wd


def workload_inputs(w, S=None):
    """Inputs of a named workload, optionally with a reduced sequence length S."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if isinstance(w, MlpWorkload) and w.gated:
        return gen_mlp_gated(w.M if S is None else S, w.K, w.N, dtype=w.dtype,
                             amp_x=w.amp_x, amp_w=w.amp_w, seed=w.seed)
    if isinstance(w, MlpWorkload):
        return gen_mlp(w.M if S is None else S, w.K, w.N, dtype=w.dtype,
                       amp_x=w.amp_x, amp_w=w.amp_w, seed=w.seed)
    S = w.S if S is None else S
    return gen_attention(w.B, w.Hq, w.Hkv, S, S, w.D, w.dtype, w.amp, w.seed)


def to_f64_numpy(t):
    """Exact widening of a CPU tensor (bf16 or f32) to a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()
