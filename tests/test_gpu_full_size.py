"""Full-size parity: the 4096-token MHA and the FFN shard compared element by
element with the float64 oracle in full, the 65536-token GQA workload on rows
covering every work item of the kernel's schedule, the explicit 16-chunk
partials-and-merge path against the fused path, and ring shares whose key and
query runs are not multiples of the kernel's tile sizes."""

import math

import numpy as np
import pytest
import torch

import oracle
from gemm_chain_amd import chain
from gemm_chain_amd.workloads import WORKLOADS, gen_attention, gen_mlp
from gpu_util import TOL_BF16, announce, device, f64, max_abs, run_threaded

pytestmark = pytest.mark.gpu


def _rows_jobs(q, k, v, b, h, rows, scale, block=256, **kw):
    return [lambda r=rows[i:i + block]: oracle.attention_rows(q, k, v, b, h, r, causal=True,
                                                              scale=scale, **kw)
            for i in range(0, len(rows), block)]


def test_mha_b2_h32_s4096_full_compare():
    """Every output row of every (batch, head) against the oracle."""
    w = WORKLOADS["attn_bf16_b2_h32_s4096_d128"]
    dev = device()
    q, k, v = gen_attention(w.B, w.Hq, w.Hkv, w.S, w.S, w.D, w.dtype, w.amp, w.seed)
    announce("full compare: MHA B2 H32 S4096")
    o, l = chain.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=True)
    torch.cuda.synchronize()
    on, ln = f64(o), l.cpu().numpy().astype(np.float64)
    qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
    allrows = np.arange(w.S)
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    jobs, where = [], []
    for b, h in heads:
        js = _rows_jobs(qn, kn, vn, b, h, allrows, w.scale, block=512)
        jobs += js
        where += [(b, h, i * 512) for i in range(len(js))]
    res = run_threaded(jobs)
    eo = el = 0.0
    for (b, h, r0), (ro, rl) in zip(where, res):
        eo = max(eo, max_abs(on[b, h, r0:r0 + len(rl)], ro))
        el = max(el, max_abs(ln[b, h, r0:r0 + len(rl)], rl))
    print(f"all {w.B * w.Hq * w.S} rows: max-abs O {eo:.3e} LSE {el:.3e}")
    assert eo <= TOL_BF16 and el <= TOL_BF16


def _gqa_rows_every_item(S, Hq, rows_per_tile=64, seed=0):
    """Per query head, one row in each pair of query tiles (t, T-1-t) the kernel takes
    as one work item, alternating between the tile, and the 32-row block inside it, that
    the row comes from, so that across heads every (tile, block) role is covered."""
    rng = np.random.default_rng(seed)
    T = S // rows_per_tile
    out = {}
    for h in range(Hq):
        rows = []
        for pr in range(T // 2):
            role = (h + pr) % 4
            t = pr if role < 2 else T - 1 - pr
            blk = role % 2
            rows.append(t * rows_per_tile + blk * 32 + int(rng.integers(32)))
        out[h] = np.array(sorted(rows), dtype=np.int64)
    return out


def test_gqa_s65536_every_work_item_and_every_block_of_one_group():
    """All 32 query heads on one row per work item; the four heads of key/value
    head 0 on one row of every 32-row block (every wave of every work item) and on
    both sides of every zigzag piece boundary."""
    w = WORKLOADS["attn_gqa_bf16_h32kv8_s65536_d128"]
    dev = device()
    q, k, v = gen_attention(w.B, w.Hq, w.Hkv, w.S, w.S, w.D, w.dtype, w.amp, w.seed)
    announce("GQA S65536: every work item")
    o, l = chain.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=True, n_chunks=w.n_chunks,
                          zigzag=w.zigzag)
    torch.cuda.synchronize()
    on, ln = o.float().cpu().numpy(), l.cpu().numpy()
    qn, kn, vn = q.float().numpy(), k.float().numpy().astype(np.float64), v.float().numpy().astype(np.float64)
    per_head = _gqa_rows_every_item(w.S, w.Hq, seed=w.seed)
    piece = w.S // (2 * w.n_chunks)
    bounds = np.array(sorted({x for p in range(1, 2 * w.n_chunks) for x in (p * piece - 1, p * piece)}))
    rng = np.random.default_rng(w.seed + 1)
    group = w.Hq // w.Hkv
    for h in range(group):
        blocks = np.arange(0, w.S, 32) + rng.integers(0, 32, size=w.S // 32)
        per_head[h] = np.unique(np.concatenate([per_head[h], blocks, bounds, [0, 1, w.S - 1]]))
    jobs, where = [], []
    for h, rows in per_head.items():
        js = _rows_jobs(qn, kn, vn, 0, h, rows, w.scale, block=128)
        jobs += js
        where += [(h, rows[i:i + 128]) for i in range(0, len(rows), 128)]
    res = run_threaded(jobs)
    eo = el = 0.0
    for (h, rows), (ro, rl) in zip(where, res):
        eo = max(eo, max_abs(on[0, h, rows], ro))
        el = max(el, max_abs(ln[0, h, rows], rl))
    n = sum(len(r) for r in per_head.values())
    print(f"{n} rows: max-abs O {eo:.3e} LSE {el:.3e}")
    assert eo <= TOL_BF16 and el <= TOL_BF16


def test_mlp_ffn_shard_m16384_full_compare():
    """The whole 16384 x 4096 output, k-major weights (the layout linear layers keep and
    the bench times); the row-major weight path must give the same bits."""
    w = WORKLOADS["mlp_bf16_m16384_k4096_n1376"]
    dev = device()
    x, w1, w2 = gen_mlp(w.M, w.K, w.N, dtype=w.dtype, amp_x=w.amp_x, amp_w=w.amp_w, seed=w.seed)
    announce("full compare: MLP 16384x4096x1376")
    xd, w1d, w2d = x.to(dev), w1.to(dev), w2.to(dev)
    o = chain.mlp_fwd(xd, w1d.t().contiguous().t(), w2d.t().contiguous().t(), act=w.act)
    o_rm = chain.mlp_fwd(xd, w1d, w2d, act=w.act)
    torch.cuda.synchronize()
    assert torch.equal(o, o_rm)
    on = f64(o)
    xn, w1n, w2n = f64(x), f64(w1), f64(w2)
    step = 2048
    res = run_threaded([lambda r0=r0: oracle.mlp(xn[r0:r0 + step], w1n, w2n, w.act)
                        for r0 in range(0, w.M, step)])
    err = max(max_abs(on[r0:r0 + step], ref) for r0, ref in zip(range(0, w.M, step), res))
    print(f"all {w.M} rows: max-abs {err:.3e}")
    assert err <= TOL_BF16


def test_gqa_sixteen_zigzag_chunks_as_partials_and_merge():
    """Reading of the 16-chunk workload: the explicit path (one chain_attn_partial per
    zigzag chunk of pieces s and 31-s, then chain_lse_merge) against the fused call and
    the oracle, GQA 32:8, at 4096 tokens."""
    dev = device()
    S, Hq, Hkv, D, C = 4096, 32, 8, 128, 16
    q, k, v = gen_attention(1, Hq, Hkv, S, S, D, "bf16", 1.0, 55)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    announce("GQA 16 zigzag chunks: partials + merge vs fused")
    of, lf = chain.attn_fwd(qd, kd, vd, causal=True, n_chunks=C, zigzag=True)
    op = torch.empty((C, 1, Hq, S, D), dtype=torch.float32, device=dev)
    lp = torch.empty((C, 1, Hq, S), dtype=torch.float32, device=dev)
    for s in range(C):
        runs = chain.zigzag_segments(S, C, s)
        kpos = torch.from_numpy(np.concatenate([np.arange(a, a + n) for a, n in runs])).to(dev)
        chain.attn_partial(qd, kd[:, :, kpos].contiguous(), vd[:, :, kpos].contiguous(), [(0, S)], runs,
                           causal=True, out=op[s], lse=lp[s])
    om, lm = chain.lse_merge(op, lp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), causal=True, scale=1 / math.sqrt(D))
    e_m, e_f = max_abs(f64(om), ro), max_abs(f64(of), ro)
    el_m, el_f = max_abs(f64(lm), rl), max_abs(f64(lf), rl)
    d = (om.float() - of.float()).abs().max().item()
    print(f"partials+merge O {e_m:.3e} LSE {el_m:.3e}; fused O {e_f:.3e} LSE {el_f:.3e}; |merge - fused| {d:.3e}")
    assert e_m <= TOL_BF16 and el_m <= TOL_BF16 and e_f <= TOL_BF16 and el_f <= TOL_BF16
    assert d <= TOL_BF16


@pytest.mark.parametrize("r", [0, 3, 7])
def test_ring_share_with_runs_of_48_tokens(r):
    """8 ranks over 768 tokens: pieces of 48, so query waves of 32 rows straddle the two
    runs of a share and every key chunk ends in a tile cut short."""
    dev = device()
    S, P, H, D = 768, 8, 4, 128
    q, k, v = gen_attention(1, H, H, S, S, D, "bf16", 1.0, 70 + r)
    qruns = chain.zigzag_segments(S, P, r)
    assert [n for _, n in qruns] == [48, 48]
    qpos = np.concatenate([np.arange(a, a + n) for a, n in qruns])
    ql = q[:, :, qpos].contiguous().to(dev)
    kd, vd = k.to(dev), v.to(dev)
    announce(f"ring share S{S} P{P} rank{r}: runs of 48")
    op = torch.empty((P, 1, H, len(qpos), D), dtype=torch.float32, device=dev)
    lp = torch.empty((P, 1, H, len(qpos)), dtype=torch.float32, device=dev)
    for i, s in enumerate([(r - i) % P for i in range(P)]):
        kruns = chain.zigzag_segments(S, P, s)
        kpos = torch.from_numpy(np.concatenate([np.arange(a, a + n) for a, n in kruns])).to(dev)
        chain.attn_partial(ql, kd[:, :, kpos].contiguous(), vd[:, :, kpos].contiguous(), qruns, kruns,
                           causal=True, out=op[i], lse=lp[i])
    o, l = chain.lse_merge(op, lp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(f64(q[:, :, qpos]), f64(k), f64(v), causal=True, scale=1 / math.sqrt(D),
                              q_pos=qpos)
    eo, el = max_abs(f64(o), ro), max_abs(f64(l), rl)
    print(f"max-abs O {eo:.3e} LSE {el:.3e}")
    assert eo <= TOL_BF16 and el <= TOL_BF16
