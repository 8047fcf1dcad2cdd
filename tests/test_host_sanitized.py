"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (argument validation, and through internal.h the schedule helpers: the
zigzag and fused key ranges, position runs, the XCD work-item remap, the tile
classification) is compiled with both sanitizers on its host pass and linked,
with the kernel objects of the regular build, into tests/sched_driver.cpp.  The
driver's results are compared with the oracle's zigzag partition and visibility
mask, and every entry point it calls with invalid arguments must return the
documented status.  Host only: no call reaches a GPU.
"""

import json
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from test_abi_cpu import _census_from_mask

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm/bin"
KERNEL_OBJS = ["attn_bwd.hip.o", "attn_mfma.hip.o", "attn_valu.hip.o", "gemm_mfma.hip.o",
               "linear_attn.hip.o", "lse_merge.hip.o"]
STATUS = {"OK": 0, "NULL": 1, "DTYPE": 2, "SHAPE": 3, "LAYOUT": 4, "ALIGN": 5, "ALIAS": 6,
          "UNSUPPORTED": 7, "WORKSPACE": 8}
EXPECTED = {
    "zigzag_uneven": "SHAPE", "zigzag_rank_out_of_range": "SHAPE", "zigzag_null": "NULL",
    "attn_null_q": "NULL", "attn_dtype": "DTYPE", "attn_heads": "SHAPE", "attn_chunks": "SHAPE",
    "attn_chunks_zigzag": "SHAPE", "attn_chunks_max": "SHAPE", "attn_align": "ALIGN", "attn_alias": "ALIAS",
    "attn_layout": "LAYOUT", "attn_headdim": "UNSUPPORTED", "attn_scale_nan": "UNSUPPORTED",
    "partial_kv_segs_cover": "SHAPE", "partial_q_segs_overlap": "SHAPE", "partial_o_dtype": "DTYPE",
    "partial_null_segs": "NULL",
    "merge_parts_mismatch": "SHAPE", "merge_alias": "ALIAS", "merge_dtype": "DTYPE",
    "mlp_workspace_small": "WORKSPACE", "mlp_act": "UNSUPPORTED", "mlp_shape": "SHAPE", "mlp_ws_alias": "ALIAS",
    "mlp_noalloc_beyond_scratch": "WORKSPACE", "gated_rowmajor_gate": "UNSUPPORTED",
    "gated_workspace_null": "WORKSPACE", "bwd_alias": "ALIAS", "bwd_workspace": "WORKSPACE",
    "lin_state_shape": "SHAPE", "lin_workspace": "WORKSPACE", "census_null_counts": "NULL",
    "census_bad_block": "SHAPE",
}


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.fixture(scope="module")
def driver_output(tmp_path_factory):
    objs = [os.path.join(ROOT, "_build", o) for o in KERNEL_OBJS]
    if not all(os.path.exists(o) for o in objs) or not os.path.exists(os.path.join(ROCM, "hipcc")):
        pytest.skip("regular build objects or hipcc missing: build the library first")
    d = tmp_path_factory.mktemp("sanitized")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "gemm_chain_amd", "csrc")]
    api = str(d / "api.o")
    # device code built as usual; AddressSanitizer and UBSan on the host pass only
    _run([os.path.join(ROCM, "hipcc"), "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          *inc, "-x", "hip", "-c", os.path.join(ROOT, "gemm_chain_amd", "csrc", "api.cpp"), "-o", api])
    drv = str(d / "driver.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    _run([os.path.join(ROCM, "amdclang++"), "-std=c++17", "-O1", "-g", *san, *inc, "-x", "hip",
          "--offload-host-only", "--offload-arch=gfx950", "-c", os.path.join(ROOT, "tests", "sched_driver.cpp"),
          "-o", drv])
    exe = str(d / "driver")
    _run([os.path.join(ROCM, "amdclang++"), *san, drv, api, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    out = _run([exe], env=env, timeout=120)
    return [json.loads(line) for line in out.splitlines() if line.startswith("{")]


def _positions(runs):
    return np.concatenate([np.arange(a, a + n) for a, n in runs if n] or [np.zeros(0, np.int64)])


def test_zigzag_segments_match_the_oracle_partition(driver_output):
    recs = [r for r in driver_output if "zz" in r]
    assert len(recs) == 1 + 8 + 3 + 8 + 16 + 8
    for r in recs:
        S, P, rank = r["zz"]
        assert r["st"] == 0
        assert np.array_equal(_positions(r["runs"]), oracle.zigzag_share_positions(S, P, rank))


def test_fused_key_ranges_visit_the_oracle_chunks_in_order(driver_output):
    recs = [r for r in driver_output if "fused" in r]
    assert len(recs) == 6
    for r in recs:
        Sk, C, zz = r["fused"]
        chunks = [oracle.zigzag_chunk_positions(Sk, C, s) if zz else oracle.natural_chunk_positions(Sk, C, s)
                  for s in range(C)]
        got = np.concatenate([np.arange(b, e) + off for b, e, off in r["ranges"]])
        assert np.array_equal(got, np.concatenate(chunks))
        assert len(r["ranges"]) == (2 * C if zz else C)


def test_position_runs_give_every_row_its_position(driver_output):
    (rp,) = [r for r in driver_output if "rowpos" in r]
    assert rp["pos"] == _positions(rp["rowpos"]).tolist()
    (rr,) = [r for r in driver_output if "runranges" in r]
    got = np.concatenate([np.arange(b, e) + off for b, e, off in rr["ranges"]])
    assert np.array_equal(got, _positions(rr["runranges"]))
    assert all(e > b for b, e, _ in rr["ranges"])          # empty runs are dropped


def test_xcd_remap_is_a_bijection(driver_output):
    recs = [r for r in driver_output if "xcd" in r]
    assert len(recs) == 15 and all(r["ok"] for r in recs)


def test_tile_censuses_match_the_oracle_mask(driver_output):
    for r in [r for r in driver_output if "census" in r]:
        Sq, bm, bn, C, zz = r["census"]
        chunks = [oracle.zigzag_chunk_positions(Sq, C, s) if zz else oracle.natural_chunk_positions(Sq, C, s)
                  for s in range(C)]
        if zz:   # tiles are cut inside each piece of a zigzag chunk
            n = Sq // (2 * C)
            chunks = [p for c in chunks for p in (c[:n], c[n:])]
        assert r["st"] == 0
        assert tuple(r["counts"]) == _census_from_mask(np.arange(Sq), chunks, True, bm, bn)
    shares = [r for r in driver_output if "share_census" in r]
    assert len(shares) == 64
    for r in shares:
        S, P, qr, kr = r["share_census"]
        qpos = oracle.zigzag_share_positions(S, P, qr)
        kpos = oracle.zigzag_share_positions(S, P, kr)
        n = S // (2 * P)
        assert r["st"] == 0
        assert tuple(r["counts"]) == _census_from_mask(qpos, [kpos[:n], kpos[n:]], True, 32, 64)


def test_invalid_arguments_return_the_documented_status(driver_output):
    got = {r["call"]: r["st"] for r in driver_output if "call" in r}
    assert set(got) == set(EXPECTED)
    for name, want in EXPECTED.items():
        assert got[name] == STATUS[want], (name, got[name], want)
