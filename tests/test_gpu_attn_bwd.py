"""GPU parity of chain_attn_bwd (dQ, dK, dV of causal / full attention with
GQA) against the float64 oracle ``oracle.attention_bwd``.

The small cases feed the backward the oracle's forward (O rounded to bf16,
LSE to f32); the full-size case feeds it the library's own forward, as in
training.  The oracle recomputes everything from Q, K, V and dO in float64.

Tolerance, element by element, from where the kernels round (Q, K, V, dO are
the same bf16 values on both sides):
  - O enters only through D_i = sum_d dO_id O_id.  With the oracle's O rounded
    to bf16 the error of D_i is the exact sum_d dO_id (O~_id - O_id); with the
    library's forward it is at most eps * sum_d |dO_id| (|O_id| + (P|V|)_id)
    (bf16 rounding of O and of the forward's P operand);
  - P (for dV) and dS (for dQ, dK) are rounded to bf16 as MFMA operands:
    relative eps each; dS also carries P_ij * (D_i error + f32 error of dP);
  - products accumulate in f32, and LSE carries f32 rounding: relative 2^-14
    covers both at these lengths;
with eps = 2^-8 (twice bf16's unit roundoff), summed over the group's query
heads for dK and dV, and the result doubled for second-order terms.  A
worst-case bound ignores cancellation, so the relative Frobenius error is also
held to 2^-7 (independent roundings of relative size <= 2^-9).
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import visible_mask
from gemm_chain_amd import chain
from gemm_chain_amd.workloads import WORKLOADS, gen_attention, gen_attention_grad
from gpu_util import announce, device, f64

pytestmark = pytest.mark.gpu

EPS = 2.0 ** -8
ACC = 2.0 ** -14


def _bounds(q, k, v, do, causal, scale, o_given=None):
    """Elementwise error bounds (dQ, dK, dV) for the kernels' rounding points.
    o_given: the bf16-rounded O the backward received (exact D_i error), or
    None when O came from the library's forward (worst-case D_i error)."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    o, lse = oracle.attention(q, k, v, causal=causal, scale=scale)
    vis = visible_mask(np.arange(S), np.arange(S), causal)
    bq, bk, bv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            Q, K, V, G, O = q[b, h], k[b, g], v[b, g], do[b, h], o[b, h]
            p = np.where(vis, np.exp(scale * (Q @ K.T) - lse[b, h][:, None]), 0.0)
            dp = G @ V.T
            ds = p * (dp - (p * dp).sum(axis=1)[:, None])
            if o_given is None:
                d_err = EPS * (np.abs(G) * (np.abs(O) + p @ np.abs(V))).sum(axis=1)
            else:
                d_err = np.abs((G * (o_given[b, h] - O)).sum(axis=1)) + ACC * (np.abs(G) * np.abs(O)).sum(axis=1)
            ds_err = EPS * np.abs(ds) + p * (d_err[:, None] + ACC * (np.abs(G) @ np.abs(V).T))
            bv[b, g] += (EPS + ACC) * (p.T @ np.abs(G))
            bq[b, h] = scale * (ds_err @ np.abs(K) + ACC * (np.abs(ds) @ np.abs(K)))
            bk[b, g] += scale * (ds_err.T @ np.abs(Q) + ACC * (np.abs(ds).T @ np.abs(Q)))
    return 2 * bq, 2 * bk, 2 * bv


def _check(name, got, ref, bound):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    err = np.abs(got - ref)
    floor = 1e-6 * max(1.0, float(np.abs(ref).max()))
    ratio = float((err / (bound + floor)).max())
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30))
    print(f"{name}: max-abs {err.max():.3e}  max|ref| {np.abs(ref).max():.3e}  "
          f"err/bound {ratio:.3f}  rel-fro {rel:.2e}")
    assert np.all(err <= bound + floor), f"{name}: error above the derived bound"
    assert rel <= 2.0 ** -7 or np.linalg.norm(ref) < 1e-6, f"{name}: relative error {rel:.2e}"


def _inputs(B, Hq, Hkv, S, D, seed, amp=1.0):
    q, k, v = gen_attention(B, Hq, Hkv, S, S, D, "bf16", amp, seed)
    do = gen_attention_grad(B, Hq, S, D, "bf16", 1.0, seed + 1000)
    return q, k, v, do


def _run(B, Hq, Hkv, S, D, causal, seed, amp=1.0):
    """Forward and backward through the library."""
    dev = device()
    q, k, v, do = _inputs(B, Hq, Hkv, S, D, seed, amp)
    announce(f"attn_bwd B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} causal{int(causal)} (library forward)")
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = chain.attn_fwd(qd, kd, vd, causal=causal)
    dq, dk, dv = chain.attn_bwd(qd, kd, vd, o, lse, dod, causal=causal)
    torch.cuda.synchronize()
    return (q, k, v, do), (dq, dk, dv)


SMALL = [
    # B, Hq, Hkv, S, D, causal
    (1, 4, 4, 300, 128, True),     # MHA, ragged tail
    (2, 8, 2, 256, 64, True),      # GQA 4:1, D 64
    (1, 6, 3, 200, 128, True),     # GQA 2:1, ragged
    (1, 3, 1, 160, 64, False),     # GQA 3:1, no mask
    (1, 4, 1, 1100, 128, True),    # many query tiles and key blocks, ragged
    (1, 2, 2, 33, 64, True),       # one partial tile
    (1, 2, 1, 1, 128, True),       # a single token
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal", SMALL)
def test_attn_bwd_small_full_compare(B, Hq, Hkv, S, D, causal):
    dev = device()
    q, k, v, do = _inputs(B, Hq, Hkv, S, D, seed=300 + S)
    qn, kn, vn, don = f64(q), f64(k), f64(v), f64(do)
    scale = 1.0 / np.sqrt(D)
    o, lse = oracle.attention(qn, kn, vn, causal=causal, scale=scale)
    ob = torch.from_numpy(o).to(torch.bfloat16)
    announce(f"attn_bwd B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} causal{int(causal)}")
    dq, dk, dv = chain.attn_bwd(q.to(dev), k.to(dev), v.to(dev), ob.to(dev),
                                torch.from_numpy(lse).to(torch.float32).to(dev), do.to(dev),
                                causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(qn, kn, vn, don, causal=causal, scale=scale)
    bq, bk, bv = _bounds(qn, kn, vn, don, causal, scale, o_given=f64(ob))
    _check("dQ", f64(dq), rq, bq)
    _check("dK", f64(dk), rk, bk)
    _check("dV", f64(dv), rv, bv)


def test_attn_bwd_full_size_heads_sampled():
    """The multi-head bf16 workload (B 2, 32 heads, S 4096, D 128) at full size;
    the oracle checks four heads of the second batch (heads are independent)."""
    w = WORKLOADS["attn_bf16_b2_h32_s4096_d128"]
    (q, k, v, do), (dq, dk, dv) = _run(w.B, w.Hq, w.Hkv, w.S, w.D, True, seed=w.seed, amp=w.amp)
    sl = (slice(1, 2), slice(8, 12))
    qn, kn, vn, don = (f64(t[sl]) for t in (q, k, v, do))
    rq, rk, rv = oracle.attention_bwd(qn, kn, vn, don, causal=True, scale=w.scale)
    bq, bk, bv = _bounds(qn, kn, vn, don, True, w.scale)
    _check("dQ", f64(dq[sl]), rq, bq)
    _check("dK", f64(dk[sl]), rk, bk)
    _check("dV", f64(dv[sl]), rv, bv)
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()


def test_attn_bwd_deterministic_and_zero_grad():
    """No atomics: two calls give identical bits; dO = 0 gives zero gradients."""
    (q, k, v, do), (dq, dk, dv) = _run(1, 8, 2, 520, 128, True, seed=11)
    dev = dq.device
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = chain.attn_fwd(qd, kd, vd)
    dq2, dk2, dv2 = chain.attn_bwd(qd, kd, vd, o, lse, dod)
    z = chain.attn_bwd(qd, kd, vd, o, lse, torch.zeros_like(dod))
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    assert all(torch.all(t == 0) for t in z)


def test_attn_bwd_strided_views_match_contiguous():
    """Inputs and outputs as [B, S, H, D] storage viewed as [B, H, S, D]."""
    dev = device()
    B, Hq, Hkv, S, D = 2, 4, 2, 200, 64
    q, k, v = gen_attention(B, Hq, Hkv, S, S, D, "bf16", 1.0, 21)
    do = gen_attention_grad(B, Hq, S, D, "bf16", 1.0, 22)
    announce("attn_bwd strided views")
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = chain.attn_fwd(qd, kd, vd)
    ref = chain.attn_bwd(qd, kd, vd, o, lse, dod)

    def bshd(t):
        return t.transpose(1, 2).contiguous().transpose(1, 2)

    outs = [torch.full((B, t.shape[2], t.shape[1], D), 9.0, device=dev).transpose(1, 2) for t in ref]
    got = chain.attn_bwd(bshd(qd), bshd(kd), bshd(vd), bshd(o), lse, bshd(dod),
                         dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
