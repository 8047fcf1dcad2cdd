#!/usr/bin/env python3
"""Throughput of the chain hot path on one MI355X.

One step = one causal GQA attention forward over the 65536-token workload
(32 query heads over 8 key/value heads, head_dim 128, bf16, 16 zigzag KV
chunks merged on chip), inputs resident in HBM before timing starts.  Prints
one JSON line: TFLOP/s (causal FLOPs = 4*B*Hq*S*S*D/2), the roofline of the
attention kernel, a record per workload (the fp32 single head, the 4096-token
MHA, one ring share with its log-sum-exp merge, the FFN shard MLP chain, and
the 65536-token GQA headline): per-step median/p10/p90, TFLOP/s, fraction of
peak, and, from the CPU-baseline leg, the max-abs error against the float64
oracle with its tolerance; secondary figures for the adjacent paths (attention
backward, gated MLP, linear attention); and the oracle timed on host threads.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary]
       [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
HEADLINE = "attn_gqa_bf16_h32kv8_s65536_d128"
TOL = {"f32": 1e-4, "bf16": 2e-2}
FLUSH_BYTES = 1 << 30         # written between cold merge calls
WARM_MS = 100.0               # warm-up of each secondary workload before timing


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


def time_region(torch, fn, steps, warmup, stream, per_step=None, before=None, warmup_ms=0.0):
    """Mean ms per call of fn over `steps` calls, HIP events on `stream`.  If
    per_step is a list, the duration of each call (events between the calls of
    the same timed region) is appended to it.  With `before`, it runs ahead of
    every call outside the timed intervals (each call is then bracketed by its
    own events and the mean is over those intervals).  Warm-up: `warmup` calls,
    continued until at least warmup_ms of wall time have passed (short kernels
    reach their steady clock only after some milliseconds of work)."""
    t0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t0) * 1e3 < warmup_ms:
        if before:
            before()
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    if before:
        marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(steps)]
        for a, b in marks:
            before()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in marks]
        if per_step is not None:
            per_step.extend(ms)
        return sum(ms) / steps
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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_threads():
    """Host threads for the oracle: the CPU share of this process, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def rate(flops, ms_list):
    s = spread(ms_list)
    tf = flops / s["median"] / 1e9
    return s, round(tf, 1), round(tf / PEAK_BF16_TFLOPS, 4)


# ---------------------------------------------------------------- GPU legs

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
    return w, (q, k, v), (o, lse), ms, flops, per_step


def config_legs(torch, chain, steps, head):
    """Timed runs of the other workloads.  Returns (records, checks): a record per
    workload, and per workload what the CPU-baseline leg needs to compare the GPU
    output with the oracle (inputs and outputs on the host)."""
    import numpy as np
    from gemm_chain_amd.workloads import WORKLOADS, gen_attention, gen_mlp
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    recs, checks = {}, {}

    # C1: single-head causal fp32 attention (launch-bound; parity is its point)
    w = WORKLOADS["attn_f32_s256_d64"]
    q, k, v = gen_attention(w.B, w.Hq, w.Hkv, w.S, w.S, w.D, w.dtype, w.amp, w.seed)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    l = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    per = []
    time_region(torch, lambda: chain.attn_fwd(qd, kd, vd, causal=True, out=o, lse=l), steps, 2, stream, per, warmup_ms=WARM_MS)
    s, tf, fr = rate(attn_flops(w.B, w.Hq, w.S, w.S, w.D), per)
    recs[w.name] = {"ms": s, "gflops": round(attn_flops(w.B, w.Hq, w.S, w.S, w.D) / s["median"] / 1e6, 2),
                    "dtype": "f32"}
    checks[w.name] = ("attn", w, (q, k, v), (o.cpu(), l.cpu()), None)

    # C2: 2 x 32 heads x 4096 tokens, bf16, one pass
    w = WORKLOADS["attn_bf16_b2_h32_s4096_d128"]
    q, k, v = gen_attention(w.B, w.Hq, w.Hkv, w.S, w.S, w.D, w.dtype, w.amp, w.seed)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    l = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    per = []
    time_region(torch, lambda: chain.attn_fwd(qd, kd, vd, causal=True, out=o, lse=l), steps, 2, stream, per, warmup_ms=WARM_MS)
    s, tf, fr = rate(attn_flops(w.B, w.Hq, w.S, w.S, w.D), per)
    recs[w.name] = {"ms": s, "tflops": tf, "frac_peak": fr, "dtype": "bf16"}
    checks[w.name] = ("attn", w, (q, k, v), (o.cpu(), l.cpu()), None)
    c2 = (qd, kd, vd, o, l)

    # C3: rank 0 of 8 over a 32768-token context: 8 partials in ring order, then the merge
    w = WORKLOADS["ring_share_bf16_h32_s32768_r0of8"]
    q, k, v = gen_attention(w.B, w.Hq, w.Hkv, w.S, w.S, w.D, w.dtype, w.amp, w.seed)
    P, r = w.ring_ranks, w.ring_rank
    qruns = chain.zigzag_segments(w.S, P, r)
    qpos = np.concatenate([np.arange(a, a + n) for a, n in qruns])
    ql = q[:, :, qpos].contiguous().to(dev)
    chunks = []
    for s_ in [(r - i) % P for i in range(P)]:
        kruns = chain.zigzag_segments(w.S, P, s_)
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

    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    per_p, per_m = [], []
    time_region(torch, partials, steps, 2, stream, per_p, warmup_ms=WARM_MS)
    time_region(torch, merge, steps, 2, stream, per_m, before=lambda: flush.fill_(1), warmup_ms=WARM_MS)
    del flush
    n = w.S // (2 * P)
    flops = 4.0 * B * H * D * (2 * P * n * n + n)       # visible pairs of the share: 2 P n^2 + n per head
    merge_bytes = P * B * H * Sl * (4 * D + 4) + B * H * Sl * (2 * D + 4)
    sp, tfp, frp = rate(flops, per_p)
    sm = spread(per_m)
    e2e = flops / (sp["median"] + sm["median"]) / 1e9
    recs[w.name] = {"ms_partials": sp, "ms_merge_cold": sm, "tflops_partials": tfp, "frac_peak_partials": frp,
                    "tflops_end_to_end": round(e2e, 1), "frac_peak_end_to_end": round(e2e / PEAK_BF16_TFLOPS, 4),
                    "merge_gbs": round(merge_bytes / sm["median"] / 1e6, 1),
                    "merge_frac_hbm": round(merge_bytes / sm["median"] / 1e6 / PEAK_HBM_GBS, 4), "dtype": "bf16"}
    checks[w.name] = ("share", w, (q, k, v), (om.cpu(), lm.cpu()), qpos)
    del chunks, ql, op, lp, om, lm

    # C4: GeLU(X.W1).W2 over the FFN shard, weights k-major (the layout linear layers keep)
    w = WORKLOADS["mlp_bf16_m16384_k4096_n1376"]
    x, w1, w2 = gen_mlp(w.M, w.K, w.N, dtype=w.dtype, amp_x=w.amp_x, amp_w=w.amp_w, seed=w.seed)
    xd = x.to(dev)
    w1c, w2c = w1.to(dev).t().contiguous().t(), w2.to(dev).t().contiguous().t()
    o = torch.empty((w.M, w.K), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(chain.mlp_workspace_bytes(w.M, w.N), dtype=torch.uint8, device=dev)
    per = []
    time_region(torch, lambda: chain.mlp_fwd(xd, w1c, w2c, act=w.act, out=o, workspace=ws), steps, 2, stream, per, warmup_ms=WARM_MS)
    s, tf, fr = rate(4.0 * w.M * w.K * w.N, per)
    w1r, w2r = w1.to(dev), w2.to(dev)
    per_r = []
    time_region(torch, lambda: chain.mlp_fwd(xd, w1r, w2r, act=w.act, out=o, workspace=ws), steps, 2, stream, per_r, warmup_ms=WARM_MS)
    sr, tfr, frr = rate(4.0 * w.M * w.K * w.N, per_r)
    chain.mlp_fwd(xd, w1c, w2c, act=w.act, out=o, workspace=ws)
    recs[w.name] = {"ms": s, "tflops": tf, "frac_peak": fr, "ms_rowmajor_w": sr, "tflops_rowmajor_w": tfr,
                    "frac_peak_rowmajor_w": frr, "dtype": "bf16"}
    checks[w.name] = ("mlp", w, (x, w1, w2), (o.cpu(),), None)
    del xd, w1c, w2c, w1r, w2r, o, ws

    # C5: the headline, timed by the main leg
    hw, hin, hout, hms, hflops, hper = head
    s, tf, fr = rate(hflops, hper)
    recs[hw.name] = {"ms": s, "tflops": tf, "frac_peak": fr, "dtype": "bf16"}
    checks[hw.name] = ("attn_rows", hw, hin, (hout[0].cpu(), hout[1].cpu()), None)
    return recs, checks, c2


def secondary(torch, chain, steps, c2):
    """Adjacent paths: attention backward of the 4096-token MHA, the gated MLP chain,
    one share of linear attention with a carried state."""
    from gemm_chain_amd.workloads import WORKLOADS, gen_attention, gen_attention_grad, gen_linear_state, gen_mlp_gated
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    out = {}

    # Backward: dQ, dK, dV from (O, LSE) and dO.  FLOPs counted as five S x S x D
    # products (S and dP recomputed, dV, dQ, dK) over the causal half: 2.5 x the forward's.
    w = WORKLOADS["attn_bf16_b2_h32_s4096_d128"]
    q, k, v, o, l = c2
    do = gen_attention_grad(w.B, w.Hq, w.S, w.D, w.dtype, 1.0, w.seed + 1000).to(dev)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    bws = torch.empty(chain.attn_bwd_workspace_bytes(w.B, w.Hq, w.S), dtype=torch.uint8, device=dev)
    per = []
    time_region(torch, lambda: chain.attn_bwd(q, k, v, o, l, do, dq=dq, dk=dk, dv=dv, workspace=bws),
                steps, 2, stream, per, warmup_ms=WARM_MS)
    s, tf, fr = rate(2.5 * attn_flops(w.B, w.Hq, w.S, w.S, w.D), per)
    out["attn_bwd_" + w.name] = {"ms": s, "tflops": tf, "frac_peak": fr}
    del do, dq, dk, dv, bws

    # Gated form (gate/up/down shards): three M x K x N products, weights k-major.
    w = WORKLOADS["mlp_gated_bf16_m16384_k4096_n1376"]
    x, wg, wu, wd = (t.to(dev) for t in gen_mlp_gated(w.M, w.K, w.N, dtype=w.dtype, amp_x=w.amp_x,
                                                      amp_w=w.amp_w, seed=w.seed))
    wg, wu, wd = (t.t().contiguous().t() for t in (wg, wu, wd))
    o = torch.empty((w.M, w.K), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(chain.mlp_workspace_bytes(w.M, w.N), dtype=torch.uint8, device=dev)
    per = []
    time_region(torch, lambda: chain.mlp_gated_fwd(x, wg, wu, wd, act=w.act, out=o, workspace=ws),
                steps, 2, stream, per, warmup_ms=WARM_MS)
    s, tf, fr = rate(6.0 * w.M * w.K * w.N, per)
    out[w.name] = {"ms": s, "tflops": tf, "frac_peak": fr}
    del x, wg, wu, wd, o, ws

    # One device's share of causal linear attention with a carried state: HBM-bound;
    # algorithmic bytes = Q, K, V read, O (f32) written, states in and out.
    w = WORKLOADS["lin_attn_bf16_h32_s32768_d128"]
    q, k, v = (t.to(dev) for t in gen_attention(w.B, w.Hq, w.Hkv, w.S, w.S, w.D, w.dtype, w.amp, w.seed))
    s_in = gen_linear_state(w.B, w.Hkv, w.D, 1.0, w.seed + 1).to(dev)
    o = torch.empty((w.B, w.Hq, w.S, w.D), dtype=torch.float32, device=dev)
    s_out = torch.empty_like(s_in)
    ws = torch.empty(chain.linear_attn_workspace_bytes(w.B, w.Hkv, w.S, w.D), dtype=torch.uint8, device=dev)
    per = []
    time_region(torch, lambda: chain.linear_attn_fwd(q, k, v, s_in=s_in, out=o, s_out=s_out, workspace=ws),
                steps, 2, stream, per, warmup_ms=WARM_MS)
    T = (w.S + 127) // 128
    flops = w.B * w.Hq * (T * 4 * w.D * 128 * 129 / 2 + 2 * w.S * w.D * w.D) + w.B * w.Hkv * 2 * w.S * w.D * w.D
    alg = 3 * q.numel() * 2 + o.numel() * 4 + 2 * s_in.numel() * 4
    s = spread(per)
    out[w.name] = {"ms": s, "tflops": round(flops / s["median"] / 1e9, 1),
                   "gbs_algorithmic": round(alg / s["median"] / 1e6, 1),
                   "frac_hbm": round(alg / s["median"] / 1e6 / PEAK_HBM_GBS, 4)}
    return out


# ---------------------------------------------------------------- CPU-baseline leg

def _headline_rows(w, seed):
    """Rows of the 65536-token check: both sides of every zigzag piece boundary and a
    seeded spread, on four heads (one per key/value head pair of the groups)."""
    import numpy as np
    piece = w.S // (2 * w.n_chunks)
    rows = {0, 1, 2, w.S - 1}
    rows.update(x for p in range(1, 2 * w.n_chunks) for x in (p * piece - 1, p * piece))
    rows.update(int(x) for x in np.random.default_rng(seed).choice(w.S, 64, replace=False))
    return np.array(sorted(rows), dtype=np.int64)


def cpu_baseline_leg(checks, budget_s=12.0):
    """The float64 oracle on host threads: (1) timed on a bounded sample of the
    headline (the cpu_baseline value), (2) the max-abs error of every workload's GPU
    output against it, with the workload's tolerance (the per-config records)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    import oracle
    W = host_threads()
    f64 = lambda t: t.to(dtype=__import__("torch").float64).numpy()  # noqa: E731

    def threaded(jobs):
        with threadpool_limits(limits=1, user_api="blas"):
            with ThreadPoolExecutor(W) as ex:
                return list(ex.map(lambda f: f(), jobs))

    def maxabs(got, ref):
        got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        fin = ~np.isneginf(ref)
        if not np.array_equal(np.isneginf(got), ~fin) or np.isnan(got).any():
            return float("inf")
        return float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0

    results = {}
    # (1) the cpu_baseline: 256-row blocks of the headline's first four query heads (one
    # key/value head) spread over the sequence, each on one thread, for about budget_s seconds
    kind, w, (q, k, v), _, _ = checks[HEADLINE]
    group = w.Hq // w.Hkv
    qn = q[:, :group].float().numpy()
    kn, vn = k[:, :1].float().numpy().astype(np.float64), v[:, :1].float().numpy().astype(np.float64)
    starts = [(h, int(x)) for h in range(group) for x in np.linspace(0, w.S - 256, 256)]
    order = [starts[i] for i in np.random.default_rng(0).permutation(len(starts))]
    done, flops, t0 = 0, 0.0, time.perf_counter()
    while done < len(order) and time.perf_counter() - t0 < budget_s:
        batch = order[done:done + W]
        threaded([lambda h=h, r0=r0: oracle.attention_rows(qn, kn, vn, 0, h, np.arange(r0, r0 + 256), causal=True,
                                                           scale=w.scale) for h, r0 in batch])
        flops += sum(4.0 * w.D * float((np.arange(r0, r0 + 256) + 1).sum()) for _, r0 in batch)
        done += len(batch)
    dt = time.perf_counter() - t0
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": W, "kind": "oracle",
            "sample": f"{done} blocks of 256 query rows of the first {group} heads spread over the {w.S}-token "
                      f"sequence, float64 numpy, one BLAS thread per host thread, {dt:.1f} s",
            "cpu_model": cpu_model(), "oracle_gflops": round(flops / dt / 1e9, 2)}

    # (2) parity of every workload's GPU output
    for name, (kind, w, inp, out, extra) in checks.items():
        t0 = time.perf_counter()
        tol = TOL[w.dtype]
        if kind == "mlp":
            x, w1, w2 = (f64(t) for t in inp)
            step = 2048
            refs = threaded([lambda r0=r0: oracle.mlp(x[r0:r0 + step], w1, w2, w.act)
                             for r0 in range(0, w.M, step)])
            on = f64(out[0])
            e = max(maxabs(on[r0:r0 + step], ref) for r0, ref in zip(range(0, w.M, step), refs))
            rec = {"max_abs_err": e, "checked": f"all {w.M} rows"}
        else:
            q, k, v = inp
            kn, vn = k.float().numpy().astype(np.float64), v.float().numpy().astype(np.float64)
            o, l = f64(out[0]), out[1].numpy().astype(np.float64)
            B, Hq, Sq, _ = q.shape
            qpos = None
            if kind == "attn":
                qn = q.float().numpy()
                heads, rows = [(b, h) for b in range(B) for h in range(Hq)], np.arange(Sq)
                what = f"all {B * Hq * Sq} rows"
            elif kind == "share":
                # the share's local rows are the global rows extra of the full sequence
                qn, qpos = q[:, :, extra].float().numpy(), extra
                heads, rows = [(0, h) for h in range(0, Hq, 4)], np.arange(0, len(extra), 8)
                what = f"every 8th local row of {len(heads)} heads"
            else:
                qn = q.float().numpy()
                rows = _headline_rows(w, w.seed)
                heads = [(0, h) for h in (0, 9, 18, 27)]
                what = f"{len(rows)} rows (zigzag piece boundaries and a spread) of 4 heads"
            jobs, where = [], []
            for b, h in heads:
                for i in range(0, len(rows), 256):
                    rr = rows[i:i + 256]
                    jobs.append(lambda b=b, h=h, rr=rr: oracle.attention_rows(
                        qn, kn, vn, b, h, rr, causal=True, scale=w.scale, q_pos=qpos))
                    where.append((b, h, rr))
            res = threaded(jobs)
            eo = max(maxabs(o[b, h, rr], ro) for (b, h, rr), (ro, _) in zip(where, res))
            el = max(maxabs(l[b, h, rr], rl) for (b, h, rr), (_, rl) in zip(where, res))
            rec = {"max_abs_err": max(eo, el), "max_abs_err_o": eo, "max_abs_err_lse": el, "checked": what}
        rec.update({"tol": tol, "pass": bool(rec["max_abs_err"] <= tol),
                    "oracle_s": round(time.perf_counter() - t0, 2)})
        results[name] = rec
    return base, results


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-secondary", action="store_true", help="time the headline only")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg (timing and parity)")
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
    head = headline(torch, chain, args.steps, args.warmup)
    w, inputs, outputs, ms, flops, per_step = head
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
        "peak_basis": "MI355X published dense bf16 MFMA 2500 TFLOP/s, HBM 8000 GB/s",
    }
    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        record["copy_calibration_bytes"] = args.copy_calibration
        del src, dst
    checks = {w.name: ("attn_rows", w, inputs, (outputs[0].cpu(), outputs[1].cpu()), None)}
    del outputs
    if not args.no_secondary:
        log("per-workload records")
        recs, checks, c2 = config_legs(torch, chain, max(5, args.steps), head)
        record["configs"] = recs
        log("secondary workloads")
        record["secondary"] = secondary(torch, chain, max(3, args.steps), c2)
        del c2
    del head
    if not args.no_cpu_baseline:
        log(f"cpu baseline and parity (oracle on {host_threads()} host threads)")
        base, parity = cpu_baseline_leg(checks)
        record["cpu_baseline"] = base
        for name, rec in parity.items():
            record.setdefault("configs", {}).setdefault(name, {}).update(rec)
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
