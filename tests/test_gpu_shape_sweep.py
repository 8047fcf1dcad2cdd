"""Property-based sweep of attention shapes against the float64 oracle:
sequence lengths around the kernel's tile edges, both head dims, MHA and GQA
4:1, one to four key chunks in natural or zigzag order.  Chunkings that do not
split the keys into equal pieces must be refused with CHAIN_ERR_SHAPE.  The
examples are drawn deterministically (derandomized) and bounded in number."""

import math

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from gemm_chain_amd import chain
from gemm_chain_amd.workloads import gen_attention
from gpu_util import TOL_BF16, announce, device, f64, max_abs

pytestmark = pytest.mark.gpu


@settings(max_examples=60, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(S=st.sampled_from([1, 17, 63, 64, 65, 128, 257]), D=st.sampled_from([64, 128]),
       group=st.sampled_from([1, 4]), n_chunks=st.sampled_from([1, 2, 4]), zigzag=st.booleans(),
       causal=st.booleans(), seed=st.integers(0, 2**16))
def test_attention_shapes_against_the_oracle(S, D, group, n_chunks, zigzag, causal, seed):
    dev = device()
    Hkv = 2
    q, k, v = gen_attention(1, Hkv * group, Hkv, S, S, D, "bf16", 1.0, seed)
    announce(f"sweep S{S} D{D} group{group} chunks{n_chunks} zz{int(zigzag)} causal{int(causal)} seed{seed}")
    pieces = 2 * n_chunks if zigzag else n_chunks
    if S % pieces:
        with pytest.raises(chain.ChainError) as e:
            chain.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, n_chunks=n_chunks, zigzag=zigzag)
        assert e.value.name == "CHAIN_ERR_SHAPE"
        return
    o, l = chain.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, n_chunks=n_chunks, zigzag=zigzag)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), causal=causal, scale=1 / math.sqrt(D))
    assert max_abs(f64(o), ro) <= TOL_BF16
    assert max_abs(f64(l), rl) <= TOL_BF16
