"""Helpers shared by the GPU tests (no arithmetic of the method here)."""

import sys

import numpy as np
import pytest
import torch

TOL_F32 = 1e-4      # max-abs bound for f32 inputs
TOL_BF16 = 2e-2     # max-abs bound for bf16 inputs with f32 accumulation


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def announce(msg):
    """Name the case before GPU work, flushed, so a fault can be attributed."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def max_abs(got, ref):
    """Max |got - ref| where both finite; -inf must match -inf exactly."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert not np.isnan(got).any(), "NaN in GPU output"
    ninf_g, ninf_r = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), "-inf pattern differs"
    fin = ~ninf_r
    if not fin.any():
        return 0.0
    return float(np.max(np.abs(got[fin] - ref[fin])))


def sample_rows(S, n, seed, extra=()):
    rng = np.random.default_rng(seed)
    rows = set(int(x) for x in rng.choice(S, size=min(n, S), replace=False))
    rows.update(r for r in (0, 1, 2, 3, S - 1, S - 2) if 0 <= r < S)
    rows.update(int(r) for r in extra if 0 <= r < S)
    return np.array(sorted(rows), dtype=np.int64)


def host_threads():
    """Worker threads for host-side reference work: the CPU share of the box, at most 16."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_threaded(jobs):
    """Run callables on host threads, one BLAS thread each, and return their results in
    order.  Threads, not processes: the test process holds the GPU, and numpy's BLAS
    calls and large ufuncs release the GIL."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(host_threads()) as ex:
            return list(ex.map(lambda f: f(), jobs))
