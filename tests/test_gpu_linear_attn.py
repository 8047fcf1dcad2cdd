"""GPU parity of chain_linear_attn_fwd (causal linear attention with a carried
key/value state) against the float64 oracle.

Tolerance, element by element, independent of how the kernels are organised:
the componentwise bound of the definition evaluated in absolute values,
  |O_gpu - O_exact|_ie <= GAMMA * (sum_{j<=i} (|q_i| . |k_j|) |v_je| + sum_d |q_id| |S_in,de|),
with GAMMA = 2^-6, which covers up to two bf16 roundings (unit roundoff 2^-9) of
any score, state or product on the way to an output element, on top of f32
accumulation; the state path is covered because |q_i S| <= sum_j (|q_i|.|k_j|)|v_j|
for S = sum_j k_j^T v_j.  It is asserted for every case, at every size.

For diagnosis only, the tests also print the error against a tighter bound
derived from where these kernels round.  The output pass takes the rows in pieces
(64 rows at D = 128, 128 at D = 64).  Inside a piece the scores q_i . k_j are
rounded to bf16 as an MFMA operand; the state before the piece is rounded to
bf16 once, from its f32 value; everything else accumulates in f32.  So, with j
running over the piece, |error of O_ie| is at most
eps * (sum_{j<=i} |s_ij| |v_je| + sum_d |q_id| |S_de|)
plus the f32 accumulation, bounded by 2^-14 times the same sums with the state's
own terms spelled out (sum_d |q_id| sum_{j before the piece} |k_jd| |v_je|), with
eps = 2^-8 (twice bf16's unit roundoff), and doubled for second-order terms.
The relative Frobenius error is also held to 2^-7.
"""

import numpy as np
import pytest
import torch

import oracle
from gemm_chain_amd import chain
from gemm_chain_amd.workloads import WORKLOADS, gen_attention, gen_linear_state
from gpu_util import announce, device, f64, sample_rows

pytestmark = pytest.mark.gpu

EPS = 2.0 ** -8
ACC = 2.0 ** -14
GAMMA = 2.0 ** -6


def _abs_bound(q, k, v, s_in, rows=None):
    """GAMMA times the definition evaluated in absolute values, at the given rows."""
    B, Hq, S, D = q.shape
    group = Hq // k.shape[1]
    rows = np.arange(S) if rows is None else np.asarray(rows)
    out = np.zeros((B, Hq, len(rows), D))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            qa = np.abs(q[b, h, rows])
            sc = (qa @ np.abs(k[b, g]).T) * (np.arange(S)[None, :] <= rows[:, None])
            out[b, h] = sc @ np.abs(v[b, g])
            if s_in is not None:
                out[b, h] += qa @ np.abs(s_in[b, g])
    return GAMMA * out


def piece_rows(D):
    """Rows the output pass takes at a time (the state is rounded once per piece)."""
    return 64 if D == 128 else 128


def _bound(q, k, v, s_in):
    """Elementwise bound on |O_gpu - O_exact| for the kernels' rounding points."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    s0 = np.zeros((B, Hkv, D, D)) if s_in is None else s_in
    piece = piece_rows(D)
    bound = np.zeros(q.shape)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            state = s0[b, g].copy()                # the state before the chunk
            astate = np.abs(s0[b, g]).copy()       # its terms in absolute value
            for t0 in range(0, S, piece):
                t1 = min(t0 + piece, S)
                qa, ka, va = np.abs(q[b, h, t0:t1]), k[b, g, t0:t1], v[b, g, t0:t1]
                sc = np.abs(q[b, h, t0:t1] @ ka.T) * np.tril(np.ones((t1 - t0, t1 - t0)))
                intra = sc @ np.abs(va)
                inter = qa @ np.abs(state)
                bound[b, h, t0:t1] = 2 * (EPS * (intra + inter) + ACC * (intra + qa @ astate))
                state += ka.T @ va
                astate += np.abs(ka).T @ np.abs(va)
    return bound


def _check(name, got, ref, bound, derived=None):
    """bound: the implementation-independent elementwise bound (asserted);
    derived: the bound from these kernels' rounding points (printed only)."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    err = np.abs(got - ref)
    floor = 1e-6 * max(1.0, float(np.abs(ref).max()))
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30))
    diag = "" if derived is None else f"  err/derived {float((err / (derived + floor)).max()):.3f}"
    print(f"{name}: max-abs {err.max():.3e}  max|ref| {np.abs(ref).max():.3e}  "
          f"err/bound {float((err / (bound + floor)).max()):.3f}{diag}  rel-fro {rel:.2e}")
    assert np.all(err <= bound + floor), f"{name}: error above the elementwise bound"
    assert rel <= 2.0 ** -7, f"{name}: relative error {rel:.2e}"


CASES = [
    # B, Hq, Hkv, S, D, with a carried state
    (1, 4, 4, 300, 128, True),     # ragged last chunk
    (2, 8, 2, 256, 64, False),     # GQA 4:1, D 64, whole chunks
    (1, 3, 1, 700, 128, True),     # GQA 3:1, six chunks
    (1, 2, 2, 4500, 64, True),     # 36 chunks, the last ragged
    (1, 64, 64, 700, 128, True),   # many heads: sums over two-chunk sub-segments, ragged
    (4, 64, 32, 1000, 64, True),   # GQA 2:1: two-chunk sub-segments, four-chunk walks
    (1, 2, 2, 129, 64, True),      # one row past a chunk
    (1, 2, 1, 1, 128, True),       # a single token
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,with_state", CASES)
def test_linear_attention_small_full_compare(B, Hq, Hkv, S, D, with_state):
    dev = device()
    q, k, v = gen_attention(B, Hq, Hkv, S, S, D, "bf16", 0.5, 500 + S)
    s_in = gen_linear_state(B, Hkv, D, 2.0, 600 + S) if with_state else None
    announce(f"linear_attn B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} state{int(with_state)}")
    o, so = chain.linear_attn_fwd(q.to(dev), k.to(dev), v.to(dev),
                                  s_in=s_in.to(dev) if with_state else None)
    torch.cuda.synchronize()
    sn = f64(s_in) if with_state else None
    ro, rs = oracle.linear_attention(f64(q), f64(k), f64(v), sn)
    _check("O", f64(o), ro, _abs_bound(f64(q), f64(k), f64(v), sn), _bound(f64(q), f64(k), f64(v), sn))
    # the state: f32 sums of exact bf16 products
    kv_abs = np.einsum("bgjd,bgje->bgde", np.abs(f64(k)), np.abs(f64(v)))
    serr = np.abs(f64(so) - rs)
    print(f"S_out: max-abs {serr.max():.3e}")
    assert np.all(serr <= ACC * (kv_abs + (np.abs(sn) if with_state else 0)) + 1e-6)


def test_linear_attention_state_passing_between_shares():
    """Two shares with the first's S_out as the second's S_in continue the sequence."""
    dev = device()
    B, H, S, D = 1, 4, 640, 128
    q, k, v = (t.to(dev) for t in gen_attention(B, H, H, S, S, D, "bf16", 0.5, 31))
    s_in = gen_linear_state(B, H, D, 1.0, 32).to(dev)
    announce("linear_attn state passing")
    whole, s_whole = chain.linear_attn_fwd(q, k, v, s_in=s_in)
    cut = 256
    o1, s1 = chain.linear_attn_fwd(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], s_in=s_in)
    o2, s2 = chain.linear_attn_fwd(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], s_in=s1)
    torch.cuda.synchronize()
    # the first share is the same computation; the second differs only by where
    # the state is rounded, so it is held to the oracle bound like the whole
    assert torch.equal(o1, whole[:, :, :cut])
    ro, rs = oracle.linear_attention(f64(q), f64(k), f64(v), f64(s_in))
    _check("O second share", f64(o2), ro[:, :, cut:],
           _abs_bound(f64(q), f64(k), f64(v), f64(s_in))[:, :, cut:],
           _bound(f64(q), f64(k), f64(v), f64(s_in))[:, :, cut:])
    assert np.max(np.abs(f64(s2) - rs)) <= 1e-3 * np.abs(rs).max()


def test_linear_attention_empty_sequence_passes_the_state():
    dev = device()
    s_in = gen_linear_state(2, 2, 64, 1.0, 33).to(dev)
    q = torch.empty(2, 4, 0, 64, dtype=torch.bfloat16, device=dev)
    k = torch.empty(2, 2, 0, 64, dtype=torch.bfloat16, device=dev)
    announce("linear_attn S = 0")
    o, so = chain.linear_attn_fwd(q, k, k.clone(), s_in=s_in)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(so, s_in)


def test_linear_attention_full_size_sampled_rows():
    """One device's 32768-token share, 32 heads of 128: sampled rows of four heads
    against the definition, and the whole state."""
    w = WORKLOADS["lin_attn_bf16_h32_s32768_d128"]
    dev = device()
    q, k, v = gen_attention(w.B, w.Hq, w.Hkv, w.S, w.S, w.D, w.dtype, w.amp, w.seed)
    s_in = gen_linear_state(w.B, w.Hkv, w.D, 1.0, w.seed + 1)
    announce("linear_attn 1x32x32768x128 full size")
    o, so = chain.linear_attn_fwd(q.to(dev), k.to(dev), v.to(dev), s_in=s_in.to(dev))
    torch.cuda.synchronize()
    rows = sample_rows(w.S, 48, w.seed, extra=(127, 128, 129, 16383, 16384))
    heads = slice(8, 12)
    qn, kn, vn, sn = f64(q[:, heads]), f64(k[:, heads]), f64(v[:, heads]), f64(s_in[:, heads])
    ref = oracle.linear_attention_rows(qn, kn, vn, rows, sn)
    got = f64(o[:, heads].cpu())[:, :, rows]
    assert np.isfinite(f64(o)).all()
    _check("O sampled rows", got, ref, _abs_bound(qn, kn, vn, sn, rows))
    rs = sn + np.einsum("bgjd,bgje->bgde", kn, vn)
    srel = np.abs(f64(so[:, heads].cpu()) - rs).max() / np.abs(rs).max()
    print(f"state: max-abs/max {srel:.2e}")
    assert srel <= 1e-5


@pytest.mark.parametrize("D", [64, 128])
def test_linear_attention_bf16_output_and_no_state_out(D):
    """A bf16 O is the f32 O rounded (same accumulation); S_out may be skipped."""
    dev = device()
    q, k, v = (t.to(dev) for t in gen_attention(1, 4, 2, 700, 700, D, "bf16", 0.5, 41))
    s_in = gen_linear_state(1, 2, D, 1.0, 42).to(dev)
    announce(f"linear_attn bf16 output D{D}")
    o32, so = chain.linear_attn_fwd(q, k, v, s_in=s_in)
    o16, none = chain.linear_attn_fwd(q, k, v, s_in=s_in, want_state=False, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert none is None and so is not None
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_linear_attention_strided_views_match_contiguous():
    """Q, K, V and O as [B, S, H, D] storage viewed as [B, H, S, D], and states
    with a padded row stride, give the contiguous call's bits."""
    dev = device()
    B, Hq, Hkv, S, D = 2, 4, 2, 300, 128
    q, k, v = (t.to(dev) for t in gen_attention(B, Hq, Hkv, S, S, D, "bf16", 0.5, 43))
    s_in = gen_linear_state(B, Hkv, D, 1.0, 44).to(dev)
    announce("linear_attn strided views")
    ref_o, ref_s = chain.linear_attn_fwd(q, k, v, s_in=s_in)

    def bshd(t):
        return t.transpose(1, 2).contiguous().transpose(1, 2)

    si_pad = torch.zeros(B, Hkv, D, D + 4, device=dev)
    si_pad[..., :D] = s_in
    so_pad = torch.full((B, Hkv, D, D + 4), 7.0, device=dev)
    o = torch.full((B, S, Hq, D), 9.0, device=dev).transpose(1, 2)
    got_o, got_s = chain.linear_attn_fwd(bshd(q), bshd(k), bshd(v), s_in=si_pad[..., :D],
                                         out=o, s_out=so_pad[..., :D])
    torch.cuda.synchronize()
    assert torch.equal(got_o, ref_o)
    assert torch.equal(got_s, ref_s)
    assert torch.all(so_pad[..., D:] == 7.0)
