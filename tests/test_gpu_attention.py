"""GPU parity of chain_attn_fwd / chain_attn_partial / chain_lse_merge against
the float64 oracle (element by element at small sizes, sampled rows at the
workloads' full sizes, and invariants that hold at any size)."""

import math

import numpy as np
import pytest
import torch

import oracle
from gemm_chain_amd import chain
from gemm_chain_amd.workloads import WORKLOADS, gen_attention
from gpu_util import TOL_BF16, TOL_F32, announce, device, f64, max_abs, sample_rows

pytestmark = pytest.mark.gpu


def _run_fwd(B, Hq, Hkv, S, D, dtype, amp, seed, n_chunks, zigzag, causal=True):
    dev = device()
    q, k, v = gen_attention(B, Hq, Hkv, S, S, D, dtype, amp, seed)
    announce(f"attn_fwd B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} {dtype} chunks{n_chunks} zz{int(zigzag)} causal{int(causal)}")
    o, l = chain.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, n_chunks=n_chunks, zigzag=zigzag)
    torch.cuda.synchronize()
    return q, k, v, o, l


def test_single_head_f32_s256_d64_full():
    w = WORKLOADS["attn_f32_s256_d64"]
    q, k, v, o, l = _run_fwd(w.B, w.Hq, w.Hkv, w.S, w.D, w.dtype, w.amp, w.seed, 1, False)
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), causal=True, scale=w.scale)
    assert o.dtype == torch.float32
    assert max_abs(f64(o), ro) <= TOL_F32
    assert max_abs(f64(l), rl) <= TOL_F32


SMALL = [
    # B, Hq, Hkv, S, D, dtype, n_chunks, zigzag, causal
    (1, 4, 4, 300, 128, "bf16", 1, False, True),     # ragged tail, MHA
    (2, 8, 2, 256, 64, "bf16", 4, True, True),       # GQA 4:1, D 64, zigzag
    (1, 4, 1, 1024, 128, "bf16", 16, True, True),    # pieces of 32 keys < tile
    (1, 2, 2, 1, 128, "bf16", 1, False, True),       # a single token
    (1, 8, 4, 200, 128, "bf16", 2, False, False),    # GQA 2:1, non-causal
    (1, 2, 1, 200, 128, "f32", 2, False, True),      # f32 path, D 128, GQA
    (2, 3, 3, 97, 64, "f32", 1, False, False),       # f32 path, non-causal
    (1, 32, 8, 640, 128, "bf16", 5, True, True),     # GQA 4:1 with zigzag pieces of 64
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,dtype,n_chunks,zigzag,causal", SMALL)
def test_attention_small_full_compare(B, Hq, Hkv, S, D, dtype, n_chunks, zigzag, causal):
    q, k, v, o, l = _run_fwd(B, Hq, Hkv, S, D, dtype, 1.0, 100 + S, n_chunks, zigzag, causal)
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), causal=causal, scale=1 / math.sqrt(D))
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert max_abs(f64(o), ro) <= tol
    assert max_abs(f64(l), rl) <= tol


def _sampled_compare(q, k, v, o, l, heads, rows_per_head, seed, scale):
    B, Hq, S, _ = q.shape
    qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
    on, ln = o.float().cpu().numpy(), l.cpu().numpy()
    worst_o = worst_l = 0.0
    for (b, h) in heads:
        rows = sample_rows(S, rows_per_head, seed + 7 * h + b)
        ro, rl = oracle.attention_rows(qn, kn, vn, b, h, rows, causal=True, scale=scale)
        worst_o = max(worst_o, max_abs(on[b, h, rows], ro))
        worst_l = max(worst_l, max_abs(ln[b, h, rows], rl))
    return worst_o, worst_l


def test_mha_bf16_b2_h32_s4096_sampled():
    w = WORKLOADS["attn_bf16_b2_h32_s4096_d128"]
    q, k, v, o, l = _run_fwd(w.B, w.Hq, w.Hkv, w.S, w.D, w.dtype, w.amp, w.seed, 1, False)
    heads = [(0, 0), (0, 17), (1, 5), (1, 31)]
    eo, el = _sampled_compare(q, k, v, o, l, heads, 96, w.seed, w.scale)
    print(f"max-abs O {eo:.3e} LSE {el:.3e}")
    assert eo <= TOL_BF16 and el <= TOL_BF16


def test_gqa_bf16_s65536_zigzag16_sampled():
    w = WORKLOADS["attn_gqa_bf16_h32kv8_s65536_d128"]
    q, k, v, o, l = _run_fwd(w.B, w.Hq, w.Hkv, w.S, w.D, w.dtype, w.amp, w.seed, w.n_chunks, w.zigzag)
    heads = [(0, 0), (0, 3), (0, 13), (0, 30)]
    eo, el = _sampled_compare(q, k, v, o, l, heads, 48, w.seed, w.scale)
    print(f"max-abs O {eo:.3e} LSE {el:.3e}")
    assert eo <= TOL_BF16 and el <= TOL_BF16


def _ring_share(q, k, v, P, r, order=None):
    """One rank's share: partials over the P zigzag chunks, then the merge."""
    dev = device()
    S = k.shape[2]
    qruns = chain.zigzag_segments(S, P, r)
    qpos = np.concatenate([np.arange(a, a + n) for a, n in qruns])
    ql = q[:, :, qpos].contiguous().to(dev)
    kd, vd = k.to(dev), v.to(dev)
    B, H, Sl, D = ql.shape
    C = P
    order = order or [(r - i) % P for i in range(P)]   # ring arrival order
    o_parts = torch.empty((C, B, H, Sl, D), dtype=torch.float32, device=dev)
    l_parts = torch.empty((C, B, H, Sl), dtype=torch.float32, device=dev)
    for i, s in enumerate(order):
        kruns = chain.zigzag_segments(S, P, s)
        kpos = torch.from_numpy(np.concatenate([np.arange(a, a + n) for a, n in kruns])).to(dev)
        kc = kd[:, :, kpos].contiguous()
        vc = vd[:, :, kpos].contiguous()
        chain.attn_partial(ql, kc, vc, qruns, kruns, causal=True, out=o_parts[i], lse=l_parts[i])
    o, l = chain.lse_merge(o_parts, l_parts, out_dtype=ql.dtype)
    torch.cuda.synchronize()
    return qpos, o, l, o_parts, l_parts


@pytest.mark.parametrize("r", range(8))
def test_ring_share_reduced_every_rank(r):
    S, P, H, D = 2048, 8, 4, 128
    q, k, v = gen_attention(1, H, H, S, S, D, "bf16", 1.0, 3)
    announce(f"ring share S{S} P{P} rank{r}")
    qpos, o, l, _, _ = _ring_share(q, k, v, P, r)
    ro, rl = oracle.attention(f64(q[:, :, qpos]), f64(k), f64(v), causal=True, scale=1 / math.sqrt(D),
                              q_pos=qpos)
    assert max_abs(f64(o), ro) <= TOL_BF16
    assert max_abs(f64(l), rl) <= TOL_BF16


def test_ring_share_s32768_rank0_sampled():
    w = WORKLOADS["ring_share_bf16_h32_s32768_r0of8"]
    q, k, v = gen_attention(w.B, w.Hq, w.Hkv, w.S, w.S, w.D, w.dtype, w.amp, w.seed)
    announce("ring share S32768 rank0 full size")
    qpos, o, l, o_parts, l_parts = _ring_share(q, k, v, w.ring_ranks, w.ring_rank)
    qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
    on, ln = o.float().cpu().numpy(), l.cpu().numpy()
    worst_o = worst_l = 0.0
    for h in (0, 9, 22, 31):
        local = sample_rows(len(qpos), 48, h, extra=(2047, 2048))
        ro, rl = oracle.attention_rows(qn, kn, vn, 0, h, qpos[local], causal=True, scale=w.scale)
        worst_o = max(worst_o, max_abs(on[0, h, local], ro))
        worst_l = max(worst_l, max_abs(ln[0, h, local], rl))
    print(f"max-abs O {worst_o:.3e} LSE {worst_l:.3e}")
    assert worst_o <= TOL_BF16 and worst_l <= TOL_BF16
    # global row 0 sees only itself: O equals V[0] exactly
    assert np.array_equal(on[0, :, 0], vn[0, :, 0])


# ------------------------------------------------------------ invariants

def test_constant_v_gives_constant_o():
    dev = device()
    q, k, _ = gen_attention(1, 4, 2, 333, 333, 128, "bf16", 1.0, 11)
    c = torch.randn(128, generator=torch.Generator().manual_seed(12)).to(torch.bfloat16)
    v = c.expand(1, 2, 333, 128).contiguous()
    announce("constant V")
    o, _ = chain.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=True, n_chunks=1)
    assert max_abs(f64(o), np.broadcast_to(f64(c), o.shape)) <= 1e-2


def test_q_zero_prefix_mean_and_log_count():
    dev = device()
    _, k, v = gen_attention(1, 2, 2, 257, 257, 64, "bf16", 1.0, 13)
    q = torch.zeros(1, 2, 257, 64, dtype=torch.bfloat16)
    announce("Q = 0")
    o, l = chain.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=True)
    vn = f64(v)[0]
    mean = np.cumsum(vn, axis=1) / np.arange(1, 258)[None, :, None]
    assert max_abs(f64(o)[0], mean) <= TOL_BF16
    assert max_abs(f64(l)[0], np.broadcast_to(np.log(np.arange(1, 258)), (2, 257))) <= 1e-5


def test_row0_equals_v0_and_chunkings_agree():
    dev = device()
    q, k, v = gen_attention(1, 8, 2, 1024, 1024, 128, "bf16", 1.0, 14)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    announce("chunkings")
    outs = [chain.attn_fwd(qd, kd, vd, causal=True, n_chunks=n, zigzag=z)
            for n, z in ((1, False), (2, False), (8, True), (16, True), (4, False))]
    ref_o, ref_l = outs[0]
    assert torch.equal(ref_o[0, :, 0], vd[0, :, 0].repeat_interleave(4, dim=0))
    for o, l in outs[1:]:
        assert (o.float() - ref_o.float()).abs().max().item() <= 1e-2
        assert (l - ref_l).abs().max().item() <= 1e-4


def test_gqa_equals_repeated_mha():
    dev = device()
    q, k, v = gen_attention(2, 16, 4, 300, 300, 128, "bf16", 1.0, 15)
    announce("GQA vs repeated MHA")
    o1, l1 = chain.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=True, n_chunks=2, zigzag=True)
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    o2, l2 = chain.attn_fwd(q.to(dev), kr.to(dev), vr.to(dev), causal=True, n_chunks=2, zigzag=True)
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-4


def test_merge_of_identical_parts_and_empty_parts():
    dev = device()
    g = torch.Generator().manual_seed(16)
    o = torch.randn(1, 2, 3, 50, 128, generator=g)
    lse = torch.randn(1, 2, 3, 50, generator=g) * 4
    parts = torch.cat([o, o]).to(dev)
    lparts = torch.cat([lse, lse]).to(dev)
    announce("merge identities")
    mo, ml = chain.lse_merge(parts, lparts, out_dtype=torch.float32)
    assert (mo.cpu() - o[0]).abs().max().item() <= 1e-6
    assert (ml.cpu() - (lse[0] + math.log(2.0))).abs().max().item() <= 1e-5
    # a part with -inf everywhere is ignored; a row with only -inf parts is (0, -inf)
    l3 = torch.stack([lse[0], torch.full_like(lse[0], -math.inf)])
    l3[:, 1, 2, 7] = -math.inf
    o3 = torch.stack([o[0], torch.randn(2, 3, 50, 128, generator=g)])
    mo, ml = chain.lse_merge(o3.to(dev), l3.to(dev), out_dtype=torch.float32)
    ref_o, ref_l = oracle.lse_merge(o3.double().numpy(), l3.double().numpy())
    assert max_abs(f64(mo), ref_o) <= 1e-5 and max_abs(f64(ml), ref_l) <= 1e-5
    assert torch.all(mo[1, 2, 7] == 0) and math.isinf(ml[1, 2, 7].item())


def test_partial_rows_with_no_visible_key():
    dev = device()
    q, k, v = gen_attention(1, 2, 2, 64, 64, 128, "bf16", 1.0, 17)
    announce("partial with invisible keys")
    o, l = chain.attn_partial(q.to(dev), k.to(dev), v.to(dev), [(0, 64)], [(100, 64)], causal=True)
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))
    # keys 50..113: rows 0..49 see nothing, later rows see a prefix
    o, l = chain.attn_partial(q.to(dev), k.to(dev), v.to(dev), [(0, 64)], [(50, 64)], causal=True)
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), causal=True, scale=1 / math.sqrt(128),
                              k_pos=np.arange(50, 114))
    assert max_abs(f64(o), ro) <= TOL_BF16 and max_abs(f64(l), rl) <= TOL_BF16
    # an empty key chunk is valid
    e = torch.empty(1, 2, 0, 128, dtype=torch.bfloat16, device=dev)
    o, l = chain.attn_partial(q.to(dev), e, e, [(0, 64)], [(0, 0)], causal=True)
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))


def test_deterministic_reruns():
    dev = device()
    q, k, v = gen_attention(1, 8, 2, 2048, 2048, 128, "bf16", 1.0, 18)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    announce("determinism")
    o1, l1 = chain.attn_fwd(qd, kd, vd, causal=True, n_chunks=4, zigzag=True)
    o2, l2 = chain.attn_fwd(qd, kd, vd, causal=True, n_chunks=4, zigzag=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_strided_views_and_empty_inputs():
    dev = device()
    q, k, v = gen_attention(1, 4, 4, 128, 128, 128, "bf16", 1.0, 19)
    # a head-major view: [B, S, H, D] storage seen as [B, H, S, D]
    qs = q.transpose(1, 2).contiguous().to(dev).transpose(1, 2)
    announce("strided views")
    o1, l1 = chain.attn_fwd(qs, k.to(dev), v.to(dev), causal=True)
    o2, l2 = chain.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    e = torch.empty(0, 4, 128, 128, dtype=torch.bfloat16, device=dev)
    o, l = chain.attn_fwd(e, e, e, causal=True)
    assert o.numel() == 0


def test_abi_errors_with_device_tensors():
    dev = device()
    q, k, v = (t.to(dev) for t in gen_attention(1, 4, 2, 128, 128, 128, "bf16", 1.0, 20))
    announce("ABI errors")
    with pytest.raises(chain.ChainError) as e:
        chain.attn_fwd(q, k, v, out=q)                                 # O aliases Q
    assert e.value.name == "CHAIN_ERR_ALIAS"
    big = torch.empty(1, 4, 128, 136, dtype=torch.bfloat16, device=dev)
    with pytest.raises(chain.ChainError) as e:
        chain.attn_fwd(big[..., 4:132], k, v)                          # 8-byte offset pointer
    assert e.value.name == "CHAIN_ERR_ALIGN"
    with pytest.raises(chain.ChainError) as e:
        chain.attn_fwd(q, k.float(), v)
    assert e.value.name == "CHAIN_ERR_DTYPE"
    with pytest.raises(chain.ChainError) as e:
        chain.attn_fwd(q, k, v, n_chunks=3)
    assert e.value.name == "CHAIN_ERR_SHAPE"
    with pytest.raises(chain.ChainError) as e:
        chain.attn_fwd(q.transpose(2, 3), k, v)
    assert e.value.name in ("CHAIN_ERR_LAYOUT", "CHAIN_ERR_SHAPE")


@pytest.mark.parametrize("C,D", [(3, 128), (5, 64), (16, 128), (1, 128), (8, 96)])
def test_merge_part_counts_against_oracle(C, D):
    """Compile-time part counts (1, 8, 16) and the generic path (3, 5), any D % 4."""
    dev = device()
    g = torch.Generator().manual_seed(60 + C)
    o = torch.randn(C, 2, 3, 77, D, generator=g)
    lse = torch.randn(C, 2, 3, 77, generator=g) * 3
    lse[0, 1, 2, :10] = -math.inf            # some parts see nothing
    lse[:, 0, 1, 5] = -math.inf              # a row that sees nothing at all
    announce(f"merge C{C} D{D}")
    mo, ml = chain.lse_merge(o.to(dev), lse.to(dev), out_dtype=torch.float32)
    ro, rl = oracle.lse_merge(o.double().numpy(), lse.double().numpy())
    assert max_abs(f64(mo), ro) <= 1e-5
    assert max_abs(f64(ml), rl) <= 1e-5
    mb, _ = chain.lse_merge(o.to(dev), lse.to(dev), out_dtype=torch.bfloat16)
    assert max_abs(f64(mb), ro) <= 2e-2


@pytest.mark.parametrize("C", [8, 6])
def test_merge_strided_parts_match_contiguous(C):
    """Partials as sequence-major views ([C, B, S, H, D] storage) and their LSE as a slice of a
    padded buffer: same bits as contiguous parts, across several batches and heads and a
    ragged last row block."""
    dev = device()
    g = torch.Generator().manual_seed(70 + C)
    B, H, S, D = 3, 5, 45, 128
    o_sm = torch.randn(C, B, S, H, D, generator=g)
    l_pad = torch.randn(C, B, H + 2, S + 3, generator=g) * 3
    l_pad[1, 2, 4, :9] = -math.inf
    announce(f"merge strided C{C}")
    o_v, l_v = o_sm.to(dev).permute(0, 1, 3, 2, 4), l_pad.to(dev)[:, :, 1:H + 1, 2:S + 2]
    mo, ml = chain.lse_merge(o_v, l_v, out_dtype=torch.float32)
    co, cl = chain.lse_merge(o_v.contiguous(), l_v.contiguous(), out_dtype=torch.float32)
    assert torch.equal(mo, co) and torch.equal(ml, cl)
    ro, rl = oracle.lse_merge(o_sm.permute(0, 1, 3, 2, 4).double().numpy(),
                              l_pad[:, :, 1:H + 1, 2:S + 2].double().numpy())
    assert max_abs(f64(mo), ro) <= 1e-5 and max_abs(f64(ml), rl) <= 1e-5


@pytest.mark.parametrize("D,n_chunks,zigzag", [(128, 5, True), (64, 1, False)])
def test_strided_kv_views_match_contiguous(D, n_chunks, zigzag):
    """K and V as head-major views ([B, S, H, D] storage): same bits as contiguous inputs."""
    dev = device()
    q, k, v = gen_attention(2, 8, 2, 320, 320, D, "bf16", 1.0, 23)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    ks = k.transpose(1, 2).contiguous().to(dev).transpose(1, 2)
    vs = v.transpose(1, 2).contiguous().to(dev).transpose(1, 2)
    assert ks.stride(2) == 2 * D and vs.stride(2) == 2 * D
    announce(f"strided K/V D{D} chunks {n_chunks} zigzag {zigzag}")
    o1, l1 = chain.attn_fwd(qd, ks, vs, causal=True, n_chunks=n_chunks, zigzag=zigzag)
    o2, l2 = chain.attn_fwd(qd, kd, vd, causal=True, n_chunks=n_chunks, zigzag=zigzag)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
