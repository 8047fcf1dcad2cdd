"""Host-side parts of bench.py (no GPU): the one-GPU rule and the per-step spread."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_step_spread_is_median_and_deciles():
    ms = [float(x) for x in range(1, 11)]   # 1 .. 10 ms
    s = bench.spread(ms)
    assert s["median"] == 5.5
    assert abs(s["p10"] - 1.9) < 1e-9 and abs(s["p90"] - 9.1) < 1e-9


def test_causal_flops_are_half_the_dense_count():
    dense = bench.attn_flops(1, 32, 65536, 65536, 128, causal=False)
    assert dense == 4.0 * 32 * 65536 * 65536 * 128
    assert bench.attn_flops(1, 32, 65536, 65536, 128) == dense / 2


def test_headline_check_rows_cover_every_zigzag_piece_boundary():
    from gemm_chain_amd.workloads import WORKLOADS
    w = WORKLOADS[bench.HEADLINE]
    rows = set(bench._headline_rows(w, w.seed).tolist())
    piece = w.S // (2 * w.n_chunks)
    for p in range(1, 2 * w.n_chunks):
        assert p * piece - 1 in rows and p * piece in rows
    assert {0, w.S - 1} <= rows and max(rows) < w.S


def test_host_threads_follow_the_affinity_mask_up_to_16():
    assert 1 <= bench.host_threads() <= min(16, len(os.sched_getaffinity(0)))
