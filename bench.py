#!/usr/bin/env python3
"""Throughput of the chain hot path on one MI355X.

One step = one causal GQA attention forward over the 65536-token workload
(32 query heads over 8 key/value heads, head_dim 128, bf16, 16 zigzag KV
chunks merged on chip), inputs resident in HBM before timing starts.  Prints
one JSON line: TFLOP/s (causal FLOPs = 4*B*Hq*S*S*D/2), the roofline of the
attention kernel, the float64 oracle timed on a bounded sample on the host,
and secondary figures for the other workloads (4096-token MHA forward and
backward, the ring share with its log-sum-exp merge, the MLP chain plain and
gated, one share of linear attention with a carried state).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary]
       [--no-cpu-baseline]
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
HEADLINE = "attn_gqa_bf16_h32kv8_s65536_d128"


def committed_traffic():
    """HBM bytes per launch of the attention kernel from the committed counter
    summary, if it was taken on the current kernel source (else None)."""
    import hashlib
    import re
    summary = os.path.join(ROOT, "profiles", "attn_gqa_s65536_d128_hbm_counters.md")
    src = os.path.join(ROOT, "gemm_chain_amd", "csrc", "attn_mfma.hip")
    try:
        text = open(summary).read()
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    t = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    h = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    if t and h and h.group(1) == digest:
        return int(t.group(1))
    return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attn_flops(B, Hq, Sq, Sk, D, causal=True):
    f = 4.0 * B * Hq * Sq * Sk * D
    return f / 2 if causal else f


def time_region(torch, fn, steps, warmup, stream, per_step=None):
    """Mean ms per call of fn over `steps` calls, HIP events on `stream`.  If
    per_step is a list, the duration of each call (events between the calls of
    the same timed region) is appended to it."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record(stream)
    for i in range(steps):
        fn()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    if per_step is not None:
        per_step.extend(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    return marks[0].elapsed_time(marks[-1]) / steps


def spread(ms):
    """median, p10 and p90 of per-step times (ms)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def device_record(torch):
    """What the numbers were measured on."""
    props = torch.cuda.get_device_properties(0)
    rec = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
           "compute_units": props.multi_processor_count,
           "memory_gib": round(props.total_memory / 2**30, 1), "rocm": torch.version.hip}
    clock = getattr(props, "clock_rate", None)
    if clock:
        rec["clock_mhz"] = round(clock / 1000)
    return rec


def headline(torch, chain, steps, warmup):
    from gemm_chain_amd.workloads import WORKLOADS, gen_attention
    w = WORKLOADS[HEADLINE]
    dev = torch.device("cuda:0")
    log(f"generating inputs for {w.name}")
    q, k, v = gen_attention(w.B, w.Hq, w.Hkv, w.S, w.S, w.D, w.dtype, w.amp, w.seed)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        chain.attn_fwd(qd, kd, vd, causal=True, n_chunks=w.n_chunks, zigzag=w.zigzag, out=o, lse=lse)

    log(f"timing {steps} steps after {warmup} warmup")
    per_step = []
    ms = time_region(torch, step, steps, warmup, stream, per_step)
    flops = attn_flops(w.B, w.Hq, w.S, w.S, w.D)
    return w, (q, k, v), ms, flops, per_step


def cpu_baseline(w, inputs, budget_s=12.0):
    """The float64 oracle on a bounded sample of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    q, k, v = inputs
    qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
    S = w.S
    blocks = [int(x) for x in np.linspace(0, S - 256, 64)]
    order = [blocks[i] for i in np.random.default_rng(0).permutation(len(blocks))]
    done, flops, t0 = 0, 0.0, time.perf_counter()
    for r0 in order:
        rows = np.arange(r0, r0 + 256)
        oracle.attention_rows(qn, kn, vn, 0, 0, rows, causal=True, scale=w.scale)
        flops += 4.0 * w.D * float((rows + 1).sum())         # visible pairs of these rows
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} blocks of 256 query rows of head 0 (positions spread over the "
                      f"{S}-token sequence), float64 numpy, {dt:.1f} s"}


def secondary(torch, chain, steps):
    """Other workloads: MHA 4096 forward and backward, ring share + merge, MLP chain
    (plain and gated), linear attention share."""
    import numpy as np
    from gemm_chain_amd.workloads import (WORKLOADS, gen_attention, gen_attention_grad, gen_linear_state,
                                          gen_mlp, gen_mlp_gated)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    out = {}

    w = WORKLOADS["attn_bf16_b2_h32_s4096_d128"]
    q, k, v = (t.to(dev) for t in gen_attention(w.B, w.Hq, w.Hkv, w.S, w.S, w.D, w.dtype, w.amp, w.seed))
    o = torch.empty_like(q)
    l = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    ms = time_region(torch, lambda: chain.attn_fwd(q, k, v, causal=True, out=o, lse=l), steps, 2, stream)
    tf = attn_flops(w.B, w.Hq, w.S, w.S, w.D) / ms / 1e9
    out[w.name] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}

    # Backward of the same attention: dQ, dK, dV from (O, LSE) and dO.  FLOPs
    # counted as five S x S x D products (S and dP recomputed, dV, dQ, dK) over
    # the causal half: 2.5 x the forward's count.
    do = gen_attention_grad(w.B, w.Hq, w.S, w.D, w.dtype, 1.0, w.seed + 1000).to(dev)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    bws = torch.empty(chain.attn_bwd_workspace_bytes(w.B, w.Hq, w.S), dtype=torch.uint8, device=dev)
    ms = time_region(torch, lambda: chain.attn_bwd(q, k, v, o, l, do, dq=dq, dk=dk, dv=dv, workspace=bws),
                     steps, 2, stream)
    tf = 2.5 * attn_flops(w.B, w.Hq, w.S, w.S, w.D) / ms / 1e9
    out["attn_bwd_" + w.name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                                 "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    del q, k, v, o, l, do, dq, dk, dv, bws

    w = WORKLOADS["ring_share_bf16_h32_s32768_r0of8"]
    q, k, v = gen_attention(w.B, w.Hq, w.Hkv, w.S, w.S, w.D, w.dtype, w.amp, w.seed)
    P, r = w.ring_ranks, w.ring_rank
    qruns = chain.zigzag_segments(w.S, P, r)
    qpos = np.concatenate([np.arange(a, a + n) for a, n in qruns])
    ql = q[:, :, qpos].contiguous().to(dev)
    chunks = []
    for s in [(r - i) % P for i in range(P)]:
        kruns = chain.zigzag_segments(w.S, P, s)
        kpos = np.concatenate([np.arange(a, a + n) for a, n in kruns])
        chunks.append((kruns, k[:, :, kpos].contiguous().to(dev), v[:, :, kpos].contiguous().to(dev)))
    B, H, Sl, D = ql.shape
    op = torch.empty((P, B, H, Sl, D), dtype=torch.float32, device=dev)
    lp = torch.empty((P, B, H, Sl), dtype=torch.float32, device=dev)
    om = torch.empty((B, H, Sl, D), dtype=torch.bfloat16, device=dev)
    lm = torch.empty((B, H, Sl), dtype=torch.float32, device=dev)

    def partials():
        for i, (kruns, kc, vc) in enumerate(chunks):
            chain.attn_partial(ql, kc, vc, qruns, kruns, causal=True, out=op[i], lse=lp[i])

    def merge():
        chain.lse_merge(op, lp, out=om, lse=lm)

    ms_p = time_region(torch, partials, steps, 2, stream)
    ms_m = time_region(torch, merge, steps * 4, 2, stream)
    # visible pairs of the share: 2 P n^2 + n per head, n = S / 2P
    n = w.S // (2 * P)
    flops = 4.0 * B * H * D * (2 * P * n * n + n)
    merge_bytes = P * B * H * Sl * (4 * D + 4) + B * H * Sl * (2 * D + 4)
    out[w.name] = {"ms_partials": round(ms_p, 4), "ms_merge": round(ms_m, 4),
                   "tflops_partials": round(flops / ms_p / 1e9, 1),
                   "tflops_end_to_end": round(flops / (ms_p + ms_m) / 1e9, 1),
                   "merge_gbs": round(merge_bytes / ms_m / 1e6, 1),
                   "merge_frac_hbm": round(merge_bytes / ms_m / 1e6 / PEAK_HBM_GBS, 4)}
    del chunks, ql, op, lp, om, lm

    w = WORKLOADS["mlp_bf16_m16384_k4096_n1376"]
    x, w1, w2 = (t.to(dev) for t in gen_mlp(w.M, w.K, w.N, dtype=w.dtype, amp_x=w.amp_x,
                                            amp_w=w.amp_w, seed=w.seed))
    o = torch.empty((w.M, w.K), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(chain.mlp_workspace_bytes(w.M, w.N), dtype=torch.uint8, device=dev)
    # Weights as linear layers store them ([out, in] row-major, i.e. column-major
    # [in, out]: k contiguous), and as row-major [in, out] arrays.
    w1c, w2c = w1.t().contiguous().t(), w2.t().contiguous().t()
    flops = 4.0 * w.M * w.K * w.N
    res = {}
    for tag, (a, b) in (("", (w1c, w2c)), ("_rowmajor_w", (w1, w2))):
        ms = time_region(torch, lambda: chain.mlp_fwd(x, a, b, act=w.act, out=o, workspace=ws), steps, 2, stream)
        res.update({"ms" + tag: round(ms, 4), "tflops" + tag: round(flops / ms / 1e9, 1),
                    "frac_peak" + tag: round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4)})
    out[w.name] = res
    del x, w1, w2, w1c, w2c, o, ws

    # Gated form (gate/up/down shards): H = act(X.Wg) * (X.Wu) in one kernel, then H.Wd;
    # weights column-major (linear-layer layout).  Three M x K x N products.
    w = WORKLOADS["mlp_gated_bf16_m16384_k4096_n1376"]
    x, wg, wu, wd = (t.to(dev) for t in gen_mlp_gated(w.M, w.K, w.N, dtype=w.dtype, amp_x=w.amp_x,
                                                      amp_w=w.amp_w, seed=w.seed))
    wg, wu, wd = (t.t().contiguous().t() for t in (wg, wu, wd))
    o = torch.empty((w.M, w.K), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(chain.mlp_workspace_bytes(w.M, w.N), dtype=torch.uint8, device=dev)
    flops = 6.0 * w.M * w.K * w.N
    ms = time_region(torch, lambda: chain.mlp_gated_fwd(x, wg, wu, wd, act=w.act, out=o, workspace=ws),
                     steps, 2, stream)
    out[w.name] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                   "frac_peak": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
    del x, wg, wu, wd, o, ws

    # One device's share of causal linear attention with a carried state (LASP):
    # HBM-bound; algorithmic bytes = Q, K, V read, O (f32) written, states in and out.
    w = WORKLOADS["lin_attn_bf16_h32_s32768_d128"]
    q, k, v = (t.to(dev) for t in gen_attention(w.B, w.Hq, w.Hkv, w.S, w.S, w.D, w.dtype, w.amp, w.seed))
    s_in = gen_linear_state(w.B, w.Hkv, w.D, 1.0, w.seed + 1).to(dev)
    o = torch.empty((w.B, w.Hq, w.S, w.D), dtype=torch.float32, device=dev)
    s_out = torch.empty_like(s_in)
    ws = torch.empty(chain.linear_attn_workspace_bytes(w.B, w.Hkv, w.S, w.D), dtype=torch.uint8, device=dev)
    ms = time_region(torch, lambda: chain.linear_attn_fwd(q, k, v, s_in=s_in, out=o, s_out=s_out, workspace=ws),
                     steps, 2, stream)
    T = (w.S + 127) // 128
    flops = w.B * w.Hq * (T * 4 * w.D * 128 * 129 / 2 + 2 * w.S * w.D * w.D) + w.B * w.Hkv * 2 * w.S * w.D * w.D
    alg = 3 * q.numel() * 2 + o.numel() * 4 + 2 * s_in.numel() * 4
    out[w.name] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                   "gbs_algorithmic": round(alg / ms / 1e6, 1),
                   "frac_hbm": round(alg / ms / 1e6 / PEAK_HBM_GBS, 4)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="also run a plain device copy of BYTES bytes (to scale HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the sharded "
              "design is described, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from gemm_chain_amd import chain
    chain.load()
    w, inputs, ms, flops, per_step = headline(torch, chain, args.steps, args.warmup)
    tflops = flops / ms / 1e9
    log(f"{w.name}: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s")
    record = {
        "metric": "causal attention fwd TFLOP/s on 1 MI355X; % of bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "seq_len": w.S, "head_dim": w.D, "causal": True, "kv_chunks": w.n_chunks,
                   "zigzag": w.zigzag, "parallelism": "single GPU"},
        "frac_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        # one step is one launch of the attention kernel, so its mean duration is ms_per_step
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": committed_traffic()},
        "step_ms": spread(per_step),
        "device": device_record(torch),
    }
    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        record["copy_calibration_bytes"] = args.copy_calibration
        del src, dst
    if not args.no_secondary:
        log("secondary workloads")
        record["secondary"] = secondary(torch, chain, max(3, args.steps))
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        record["cpu_baseline"] = cpu_baseline(w, inputs)
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
