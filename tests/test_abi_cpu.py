"""The C ABI without a GPU: exports, validation status codes, host schedule.

Every call here either is a pure host helper or fails validation before any
launch (descriptors carry fake, never-dereferenced device addresses), so no
GPU work is attempted.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from gemm_chain_amd import chain

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def header_functions():
    text = open(os.path.join(ROOT, "include", "chain.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(chain_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(chain.library_path()):
        pytest.skip("libchain.so not built")
    return chain.load()


def td(shape, dtype=chain.BF16, data=FAKE, stride=None):
    t = chain.ChainTensor()
    t.data = data
    t.dtype = dtype
    t.ndim = len(shape)
    if stride is None:
        stride, acc = [], 1
        for n in reversed(shape):
            stride.insert(0, acc)
            acc *= n
    for i, (n, s) in enumerate(zip(shape, stride)):
        t.shape[i] = n
        t.stride[i] = s
    return t


def test_every_declared_function_is_exported(lib):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert lib.chain_version() == 100
    assert lib.chain_status_str(0) == b"CHAIN_OK"
    assert lib.chain_status_str(6) == b"CHAIN_ERR_ALIAS"


def _attn(lib, Q, K, V, O, L, causal=1, scale=0.125, n_chunks=1, zigzag=0):
    P = ctypes.byref
    return lib.chain_attn_fwd(P(Q), P(K), P(V), P(O), P(L), causal, scale, n_chunks, zigzag, None)


def _valid(B=1, Hq=4, Hkv=2, S=256, D=64, dt=chain.BF16, odt=None):
    es = 4 if dt == chain.F32 else 2
    base = FAKE
    sz = B * Hq * S * D * es
    Q = td([B, Hq, S, D], dt, base)
    K = td([B, Hkv, S, D], dt, base + 1 * 2 ** 30)
    V = td([B, Hkv, S, D], dt, base + 2 * 2 ** 30)
    O = td([B, Hq, S, D], dt if odt is None else odt, base + 3 * 2 ** 30)
    L = td([B, Hq, S], chain.F32, base + 4 * 2 ** 30)
    assert sz < 2 ** 30
    return Q, K, V, O, L


CODES = {n: i for i, n in enumerate(chain.STATUS)}


def test_attn_rows_of_a_head_must_span_under_2gib(lib):
    """bf16 kernels address a head's key/value rows with 32-bit byte offsets."""
    Q, K, V, O, L = _valid()
    far = FAKE + 2 ** 44
    for stride_s, ok in ((2 ** 22, True), (2 ** 23, False)):
        Kw = td([1, 2, 256, 64], chain.BF16, far, stride=[2 ** 40, 2 ** 31, stride_s, 1])
        Vw = td([1, 2, 256, 64], chain.BF16, far + 2 ** 42, stride=[2 ** 40, 2 ** 31, stride_s, 1])
        rc = _attn(lib, Q, Kw, Vw, O, L, scale=-1.0)   # a valid span fails later, at the scale check
        assert rc == CODES["CHAIN_ERR_UNSUPPORTED"]
        msg = lib.chain_last_error().decode()
        assert ("2 GiB" in msg) != ok, (stride_s, msg)


def test_attn_validation_codes(lib):
    Q, K, V, O, L = _valid()
    P = ctypes.byref
    assert lib.chain_attn_fwd(None, P(K), P(V), P(O), P(L), 1, 0.1, 1, 0, None) == CODES["CHAIN_ERR_NULL"]
    Qn = _valid()[0]
    Qn.data = None
    assert _attn(lib, Qn, K, V, O, L) == CODES["CHAIN_ERR_NULL"]
    Kf = _valid(dt=chain.F32)[1]
    assert _attn(lib, Q, Kf, V, O, L) == CODES["CHAIN_ERR_DTYPE"]
    Lb = td([1, 4, 256], chain.BF16, FAKE + 4 * 2 ** 30)
    assert _attn(lib, Q, K, V, O, Lb) == CODES["CHAIN_ERR_DTYPE"]
    Ob = _valid(odt=chain.F32)[3]
    assert _attn(lib, Q, K, V, Ob, L) == CODES["CHAIN_ERR_DTYPE"]
    K3 = td([1, 3, 256, 64], chain.BF16, FAKE + 2 ** 30)
    V3 = td([1, 3, 256, 64], chain.BF16, FAKE + 2 * 2 ** 30)
    assert _attn(lib, Q, K3, V3, O, L) == CODES["CHAIN_ERR_SHAPE"]            # 4 % 3
    Os = td([1, 4, 255, 64], chain.BF16, FAKE + 3 * 2 ** 30)
    assert _attn(lib, Q, K, V, Os, L) == CODES["CHAIN_ERR_SHAPE"]
    Qs = td([1, 4, 256, 64], chain.BF16, FAKE, stride=[4 * 256 * 128, 256 * 128, 128, 2])
    assert _attn(lib, Qs, K, V, O, L) == CODES["CHAIN_ERR_LAYOUT"]
    Qa = td([1, 4, 256, 64], chain.BF16, FAKE + 8)
    assert _attn(lib, Qa, K, V, O, L) == CODES["CHAIN_ERR_ALIGN"]
    Qr = td([1, 4, 256, 64], chain.BF16, FAKE, stride=[4 * 256 * 68, 256 * 68, 68, 1])
    assert _attn(lib, Qr, K, V, O, L) == CODES["CHAIN_ERR_ALIGN"]             # 136-byte rows
    Oal = td([1, 4, 256, 64], chain.BF16, FAKE + 4096)                           # overlaps Q
    assert _attn(lib, Q, K, V, Oal, L) == CODES["CHAIN_ERR_ALIAS"]
    Q96, K96, V96, O96, L96 = _valid(D=96)
    assert _attn(lib, Q96, K96, V96, O96, L96) == CODES["CHAIN_ERR_UNSUPPORTED"]
    assert _attn(lib, Q, K, V, O, L, scale=0.0) == CODES["CHAIN_ERR_UNSUPPORTED"]
    assert _attn(lib, Q, K, V, O, L, scale=float("nan")) == CODES["CHAIN_ERR_UNSUPPORTED"]
    assert _attn(lib, Q, K, V, O, L, n_chunks=3) == CODES["CHAIN_ERR_SHAPE"]      # 256 % 3
    assert _attn(lib, Q, K, V, O, L, n_chunks=256, zigzag=1) == CODES["CHAIN_ERR_SHAPE"]
    assert _attn(lib, Q, K, V, O, L, n_chunks=0) == CODES["CHAIN_ERR_SHAPE"]
    assert _attn(lib, Q, K, V, O, L, n_chunks=65) == CODES["CHAIN_ERR_SHAPE"]
    Kl, Vl = td([1, 2, 512, 64], chain.BF16, FAKE + 2 ** 30), td([1, 2, 512, 64], chain.BF16, FAKE + 2 * 2 ** 30)
    assert _attn(lib, Q, Kl, Vl, O, L, causal=1) == CODES["CHAIN_ERR_SHAPE"]    # causal needs Sk == Sq
    assert b"multiple" in lib.chain_last_error() or lib.chain_last_error() != b""


def test_partial_validation_codes(lib):
    Q, K, V, _, L = _valid()
    O = td([1, 4, 256, 64], chain.F32, FAKE + 3 * 2 ** 30)
    P = ctypes.byref
    good = chain.segs([(0, 128), (1000, 128)])
    assert lib.chain_attn_partial(P(Q), P(K), P(V), P(O), P(L), 1, 0.1, P(good), None, None) == CODES["CHAIN_ERR_NULL"]
    short = chain.segs([(0, 100)])
    assert lib.chain_attn_partial(P(Q), P(K), P(V), P(O), P(L), 1, 0.1, P(good), P(short), None) == CODES["CHAIN_ERR_SHAPE"]
    overlapping = chain.segs([(0, 200), (100, 56)])
    assert lib.chain_attn_partial(P(Q), P(K), P(V), P(O), P(L), 1, 0.1, P(overlapping), P(good), None) == CODES["CHAIN_ERR_SHAPE"]
    Ob = td([1, 4, 256, 64], chain.BF16, FAKE + 3 * 2 ** 30)
    assert lib.chain_attn_partial(P(Q), P(K), P(V), P(Ob), P(L), 1, 0.1, P(good), P(good), None) == CODES["CHAIN_ERR_DTYPE"]


def test_merge_and_mlp_validation_codes(lib):
    P = ctypes.byref
    Op = td([8, 1, 4, 256, 64], chain.F32, FAKE)
    Lp = td([8, 1, 4, 256], chain.F32, FAKE + 2 ** 30)
    O = td([1, 4, 256, 64], chain.BF16, FAKE + 2 * 2 ** 30)
    L = td([1, 4, 256], chain.F32, FAKE + 3 * 2 ** 30)
    Lpb = td([8, 1, 4, 256], chain.BF16, FAKE + 2 ** 30)
    assert lib.chain_lse_merge(P(Op), P(Lpb), P(O), P(L), None) == CODES["CHAIN_ERR_DTYPE"]
    Lp7 = td([7, 1, 4, 256], chain.F32, FAKE + 2 ** 30)
    assert lib.chain_lse_merge(P(Op), P(Lp7), P(O), P(L), None) == CODES["CHAIN_ERR_SHAPE"]
    Oal = td([1, 4, 256, 64], chain.BF16, FAKE + 64)
    assert lib.chain_lse_merge(P(Op), P(Lp), P(Oal), P(L), None) == CODES["CHAIN_ERR_ALIAS"]
    # more 8-row blocks of (batch, head) rows than 32-bit workgroup numbers (2^30 + 1 heads of
    # 9 rows: 9.7e9 rows in 2^31 + 2 blocks), or more heads than 32 bits: refused before any launch
    for heads, S in [(2 ** 30 + 1, 9), (2 ** 31, 1)]:
        Oh = td([1, 1, heads, S, 4], chain.F32, FAKE)
        Lh = td([1, 1, heads, S], chain.F32, FAKE + 2 ** 44)
        Mo = td([1, heads, S, 4], chain.F32, FAKE + 2 ** 45)
        assert lib.chain_lse_merge(P(Oh), P(Lh), P(Mo), None, None) == CODES["CHAIN_ERR_UNSUPPORTED"]

    X = td([512, 256], chain.BF16, FAKE)
    W1 = td([256, 128], chain.BF16, FAKE + 2 ** 30)
    W2 = td([128, 256], chain.BF16, FAKE + 2 * 2 ** 30)
    Om = td([512, 256], chain.BF16, FAKE + 3 * 2 ** 30)
    need = lib.chain_mlp_workspace_bytes(512, 128, chain.BF16)
    assert need == 512 * 128 * 2
    ws = FAKE + 4 * 2 ** 30
    assert lib.chain_mlp_fwd(P(X), P(W1), P(W2), P(Om), 0, ws, need - 1, None) == CODES["CHAIN_ERR_WORKSPACE"]
    assert lib.chain_mlp_fwd(P(X), P(W1), P(W2), P(Om), 0, None, need, None) == CODES["CHAIN_ERR_WORKSPACE"]
    assert lib.chain_mlp_fwd(P(X), P(W1), P(W2), P(Om), 7, ws, need, None) == CODES["CHAIN_ERR_UNSUPPORTED"]
    W1b = td([255, 128], chain.BF16, FAKE + 2 ** 30)
    assert lib.chain_mlp_fwd(P(X), P(W1b), P(W2), P(Om), 0, ws, need, None) == CODES["CHAIN_ERR_SHAPE"]
    W1f = td([256, 128], chain.F32, FAKE + 2 ** 30)
    assert lib.chain_mlp_fwd(P(X), P(W1f), P(W2), P(Om), 0, ws, need, None) == CODES["CHAIN_ERR_DTYPE"]
    assert lib.chain_mlp_fwd(P(X), P(W1), P(W2), P(Om), 0, FAKE + 256, need, None) == CODES["CHAIN_ERR_ALIAS"]
    # Weights may be row- or column-major, but one dimension must be contiguous.
    W1s = td([256, 128], chain.BF16, FAKE + 2 ** 30, stride=[256, 2])
    assert lib.chain_mlp_fwd(P(X), P(W1s), P(W2), P(Om), 0, ws, need, None) == CODES["CHAIN_ERR_LAYOUT"]
    W1c = td([256, 128], chain.BF16, FAKE + 2 ** 30, stride=[1, 264])   # column-major, aligned
    W1m = td([256, 128], chain.BF16, FAKE + 2 ** 30, stride=[1, 257])   # column stride not 16-byte
    assert lib.chain_mlp_fwd(P(X), P(W1m), P(W2), P(Om), 0, ws, need, None) == CODES["CHAIN_ERR_ALIGN"]
    W1w = td([256, 128], chain.BF16, FAKE + 2 ** 40, stride=[1, 2 ** 25 + 8])
    assert lib.chain_mlp_fwd(P(X), P(W1w), P(W2), P(Om), 0, ws, need, None) == CODES["CHAIN_ERR_UNSUPPORTED"]
    # A valid column-major weight passes validation (the error comes from elsewhere).
    assert lib.chain_mlp_fwd(P(X), P(W1c), P(W2), P(Om), 7, ws, need, None) == CODES["CHAIN_ERR_UNSUPPORTED"]
    Xc = td([512, 256], chain.BF16, FAKE, stride=[1, 512])               # X must be row-major
    assert lib.chain_mlp_fwd(P(Xc), P(W1), P(W2), P(Om), 0, ws, need, None) == CODES["CHAIN_ERR_LAYOUT"]


@pytest.mark.parametrize("S,P", [(32, 1), (256, 8), (32768, 8), (96, 3)])
def test_zigzag_segments_match_oracle(lib, S, P):
    for r in range(P):
        runs = chain.zigzag_segments(S, P, r)
        pos = np.concatenate([np.arange(a, a + n) for a, n in runs])
        assert np.array_equal(pos, oracle.zigzag_share_positions(S, P, r))
    with pytest.raises(chain.ChainError):
        chain.zigzag_segments(S + 1, P, 0)
    with pytest.raises(chain.ChainError):
        chain.zigzag_segments(S, P, P)


def _census_from_mask(qpos, kranges, causal, bm, bn):
    """Tile classes recomputed from the oracle's visibility mask."""
    full = diag = skip = 0
    for r0 in range(0, len(qpos), bm):
        qp = qpos[r0:r0 + bm]
        for kpos in kranges:
            for k0 in range(0, len(kpos), bn):
                kp = kpos[k0:k0 + bn]
                vis = oracle.visible_mask(qp, kp, causal)
                if not vis.any():
                    skip += 1
                elif vis.all() and len(kp) == bn:
                    full += 1
                else:
                    diag += 1
    return full, diag, skip


@pytest.mark.parametrize("Sq,bm,bn,n_chunks,zigzag", [
    (256, 32, 64, 1, False), (256, 32, 64, 4, True), (300, 32, 64, 1, False),
    (512, 128, 64, 8, True), (1024, 32, 64, 16, True), (192, 32, 64, 3, False)])
def test_tile_census_fused_matches_mask(lib, Sq, bm, bn, n_chunks, zigzag):
    ranges = [oracle.zigzag_chunk_positions(Sq, n_chunks, s) if zigzag else
              oracle.natural_chunk_positions(Sq, n_chunks, s) for s in range(n_chunks)]
    if zigzag:  # the kernels cut tiles inside each piece of a zigzag chunk
        n = Sq // (2 * n_chunks)
        ranges = [piece for r in ranges for piece in (r[:n], r[n:])]
    got = chain.tile_census(Sq, Sq, n_chunks=n_chunks, zigzag=zigzag, block_m=bm, block_n=bn)
    assert got == _census_from_mask(np.arange(Sq), ranges, True, bm, bn)
    # every visible pair is covered by a FULL or DIAG tile, none by a SKIP tile
    assert got[0] + got[1] + got[2] == sum(-(-Sq // bm) * -(-len(r) // bn) for r in ranges)


def test_tile_census_ring_share(lib):
    S, P = 2048, 8
    qruns = chain.zigzag_segments(S, P, 0)
    qpos = oracle.zigzag_share_positions(S, P, 0)
    for s in range(P):
        kruns = chain.zigzag_segments(S, P, s)
        kpos = oracle.zigzag_chunk_positions(S, P, s)
        n = S // (2 * P)
        got = chain.tile_census(len(qpos), len(kpos), q_pos=qruns, kv_pos=kruns, block_m=32, block_n=64)
        assert got == _census_from_mask(qpos, [kpos[:n], kpos[n:]], True, 32, 64)


def _bwd_set(B=1, Hq=4, Hkv=2, S=256, D=64):
    G = 2 ** 30
    Q, K, V, O, L = _valid(B, Hq, Hkv, S, D)
    dO = td([B, Hq, S, D], chain.BF16, FAKE + 5 * G)
    dQ = td([B, Hq, S, D], chain.F32, FAKE + 6 * G)
    dK = td([B, Hkv, S, D], chain.F32, FAKE + 7 * G)
    dV = td([B, Hkv, S, D], chain.F32, FAKE + 8 * G)
    return dict(Q=Q, K=K, V=V, O=O, L=L, dO=dO, dQ=dQ, dK=dK, dV=dV), FAKE + 9 * G


def _bwd(lib, t, ws, ws_bytes, **over):
    t = dict(t, **over)
    P = ctypes.byref
    return lib.chain_attn_bwd(P(t["Q"]), P(t["K"]), P(t["V"]), P(t["O"]), P(t["L"]), P(t["dO"]),
                              P(t["dQ"]), P(t["dK"]), P(t["dV"]), 1, 0.125, ws, ws_bytes, None)


def test_attn_bwd_validation_codes(lib):
    t, ws = _bwd_set()
    need = lib.chain_attn_bwd_workspace_bytes(1, 4, 256)
    assert need == 4 * 256 * 8                              # rows padded to 64, 8 bytes each
    assert lib.chain_attn_bwd_workspace_bytes(1, 3, 5) == 3 * 64 * 8
    assert lib.chain_attn_bwd_workspace_bytes(-1, 3, 5) == 0
    G = 2 ** 30
    # Everything else valid: the missing or short workspace is what fails.
    assert _bwd(lib, t, None, need) == CODES["CHAIN_ERR_WORKSPACE"]
    assert _bwd(lib, t, ws, need - 1) == CODES["CHAIN_ERR_WORKSPACE"]
    assert _bwd(lib, t, ws + 16, need) == CODES["CHAIN_ERR_ALIGN"]
    assert _bwd(lib, t, FAKE + 5 * G + 256, need) == CODES["CHAIN_ERR_ALIAS"]      # inside dO
    assert _bwd(lib, t, FAKE + 7 * G + 1024, need) == CODES["CHAIN_ERR_ALIAS"]     # inside dK
    assert _bwd(lib, t, ws, need, dQ=td([1, 4, 256, 64], chain.BF16, FAKE + 6 * G)) == CODES["CHAIN_ERR_DTYPE"]
    assert _bwd(lib, t, ws, need, dO=td([1, 4, 256, 64], chain.F32, FAKE + 5 * G)) == CODES["CHAIN_ERR_DTYPE"]
    f32 = _valid(dt=chain.F32)
    assert _bwd(lib, t, ws, need, Q=f32[0], K=f32[1], V=f32[2], O=f32[3]) == CODES["CHAIN_ERR_DTYPE"]
    assert _bwd(lib, t, ws, need, dK=td([1, 2, 255, 64], chain.F32, FAKE + 7 * G)) == CODES["CHAIN_ERR_SHAPE"]
    assert _bwd(lib, t, ws, need, dO=td([1, 4, 255, 64], chain.BF16, FAKE + 5 * G)) == CODES["CHAIN_ERR_SHAPE"]
    assert _bwd(lib, t, ws, need, dQ=td([1, 4, 256, 64], chain.F32, FAKE + 2048)) == CODES["CHAIN_ERR_ALIAS"]
    assert _bwd(lib, t, ws, need, dV=td([1, 2, 256, 64], chain.F32, FAKE + 7 * G + 4096)) == CODES["CHAIN_ERR_ALIAS"]
    assert _bwd(lib, t, ws, need, dV=td([1, 2, 256, 64], chain.F32, FAKE + 8 * G + 8)) == CODES["CHAIN_ERR_ALIGN"]
    assert _bwd(lib, t, ws, need, dO=td([1, 4, 256, 64], chain.BF16, FAKE + 5 * G,
                                        stride=[4 * 256 * 68, 256 * 68, 68, 1])) == CODES["CHAIN_ERR_ALIGN"]
    # keys must match queries
    t2, _ = _bwd_set()
    t2["K"] = td([1, 2, 128, 64], chain.BF16, FAKE + G)
    t2["V"] = td([1, 2, 128, 64], chain.BF16, FAKE + 2 * G)
    t2["dK"] = td([1, 2, 128, 64], chain.F32, FAKE + 7 * G)
    t2["dV"] = td([1, 2, 128, 64], chain.F32, FAKE + 8 * G)
    assert _bwd(lib, t2, ws, need) == CODES["CHAIN_ERR_SHAPE"]
    # one head's query rows must span less than 2^31 bytes (32-bit buffer offsets)
    Qw = td([1, 4, 256, 64], chain.BF16, FAKE + 2 ** 44, stride=[4 * 256 * 2 ** 23, 256 * 2 ** 23, 2 ** 23, 1])
    Ow = td([1, 4, 256, 64], chain.BF16, FAKE + 2 ** 45, stride=[4 * 256 * 2 ** 23, 256 * 2 ** 23, 2 ** 23, 1])
    assert _bwd(lib, t, ws, need, Q=Qw) == CODES["CHAIN_ERR_UNSUPPORTED"]
    assert _bwd(lib, t, ws, need, dO=Ow) == CODES["CHAIN_ERR_UNSUPPORTED"]
    t3, _ = _bwd_set(D=96)
    assert _bwd(lib, t3, ws, need) == CODES["CHAIN_ERR_UNSUPPORTED"]
    # Empty sequence: valid, nothing launched.
    t0, _ = _bwd_set(S=0)
    assert _bwd(lib, t0, None, 0) == CODES["CHAIN_OK"]


def test_mlp_gated_validation_codes(lib):
    P = ctypes.byref
    G = 2 ** 30
    X = td([512, 256], chain.BF16, FAKE)
    Wg = td([256, 128], chain.BF16, FAKE + G, stride=[1, 264])        # column-major
    Wu = td([256, 128], chain.BF16, FAKE + 2 * G, stride=[1, 264])
    Wd = td([128, 256], chain.BF16, FAKE + 3 * G)
    O = td([512, 256], chain.BF16, FAKE + 4 * G)
    need = lib.chain_mlp_workspace_bytes(512, 128, chain.BF16)
    ws = FAKE + 5 * G

    def call(x=X, wg=Wg, wu=Wu, wd=Wd, o=O, act=3, w=ws, n=need):
        return lib.chain_mlp_gated_fwd(P(x), P(wg), P(wu), P(wd), P(o), act, w, n, None)

    # everything else valid: the missing workspace is what fails
    assert call(w=None) == CODES["CHAIN_ERR_WORKSPACE"]
    assert call(n=need - 1) == CODES["CHAIN_ERR_WORKSPACE"]
    assert call(act=9, w=None) == CODES["CHAIN_ERR_UNSUPPORTED"]
    # gate/up weights share one layout (row- or column-major) and their strides
    assert call(wg=td([256, 128], chain.BF16, FAKE + G), w=None) == CODES["CHAIN_ERR_UNSUPPORTED"]
    assert call(wu=td([256, 128], chain.BF16, FAKE + 2 * G, stride=[1, 272]), w=None) == CODES["CHAIN_ERR_UNSUPPORTED"]
    rg, ru = td([256, 128], chain.BF16, FAKE + G), td([256, 128], chain.BF16, FAKE + 2 * G)
    assert call(wg=rg, wu=ru, w=None) == CODES["CHAIN_ERR_WORKSPACE"]   # both row-major: valid
    assert call(wg=rg, wu=td([256, 128], chain.BF16, FAKE + 2 * G, stride=[136, 1]),
                w=None) == CODES["CHAIN_ERR_UNSUPPORTED"]
    # row-major rows whose band passes 2^31 bytes (checked before any launch)
    # (the two bands overlap each other, which inputs may, and end below O)
    far = 2 ** 22 + 2 ** 16
    assert call(wg=td([256, 128], chain.BF16, FAKE + G, stride=[far, 1]),
                wu=td([256, 128], chain.BF16, FAKE + G + 1024, stride=[far, 1])) == CODES["CHAIN_ERR_UNSUPPORTED"]
    assert call(wu=td([256, 136], chain.BF16, FAKE + 2 * G, stride=[1, 264]), w=None) == CODES["CHAIN_ERR_SHAPE"]
    assert call(wd=td([128, 256], chain.F32, FAKE + 3 * G), w=None) == CODES["CHAIN_ERR_DTYPE"]
    f32 = dict(x=td([512, 256], chain.F32, FAKE), wg=td([256, 128], chain.F32, FAKE + G, stride=[1, 264]),
               wu=td([256, 128], chain.F32, FAKE + 2 * G, stride=[1, 264]), wd=td([128, 256], chain.F32, FAKE + 3 * G))
    assert call(w=None, **f32) == CODES["CHAIN_ERR_UNSUPPORTED"]
    assert call(o=td([512, 256], chain.BF16, FAKE + G + 64), w=None) == CODES["CHAIN_ERR_ALIAS"]
    assert call(w=FAKE + 2 * G + 1024) == CODES["CHAIN_ERR_ALIAS"]
    assert call(w=ws + 16) == CODES["CHAIN_ERR_ALIGN"]
    assert call(x=td([512, 250], chain.BF16, FAKE, stride=[256, 1]), wg=td([250, 128], chain.BF16, FAKE + G, stride=[1, 264]),
                wu=td([250, 128], chain.BF16, FAKE + 2 * G, stride=[1, 264]), w=None) == CODES["CHAIN_ERR_UNSUPPORTED"]


def test_linear_attn_validation_codes(lib):
    P = ctypes.byref
    G = 2 ** 30
    Q = td([1, 4, 256, 128], chain.BF16, FAKE)
    K = td([1, 2, 256, 128], chain.BF16, FAKE + G)
    V = td([1, 2, 256, 128], chain.BF16, FAKE + 2 * G)
    O = td([1, 4, 256, 128], chain.F32, FAKE + 3 * G)
    Si = td([1, 2, 128, 128], chain.F32, FAKE + 4 * G)
    So = td([1, 2, 128, 128], chain.F32, FAKE + 5 * G)
    need = lib.chain_linear_attn_workspace_bytes(1, 2, 256, 128)
    # two heads x two one-chunk sub-segments: an f32 sum and an f32 start state each
    assert need == 2 * (2 * 2 * 128 * 128 * 4)
    # many heads: one sub-segment per head
    assert lib.chain_linear_attn_workspace_bytes(4, 128, 100000, 64) == 2 * (4 * 128 * 64 * 64 * 4)
    ws = FAKE + 6 * G

    def call(q=Q, k=K, v=V, o=O, si=Si, so=So, w=ws, n=need):
        return lib.chain_linear_attn_fwd(P(q), P(k), P(v), P(o), P(si) if si else None,
                                         P(so) if so else None, w, n, None)

    assert call(w=None) == CODES["CHAIN_ERR_WORKSPACE"]
    assert call(n=need - 1) == CODES["CHAIN_ERR_WORKSPACE"]
    assert call(w=ws + 64) == CODES["CHAIN_ERR_ALIGN"]
    assert call(w=FAKE + 2 * G + 4096) == CODES["CHAIN_ERR_ALIAS"]
    assert call(si=None, so=None, w=None) == CODES["CHAIN_ERR_WORKSPACE"]
    assert call(q=td([1, 4, 256, 128], chain.F32, FAKE), w=None) == CODES["CHAIN_ERR_DTYPE"]
    assert call(si=td([1, 2, 128, 128], chain.BF16, FAKE + 4 * G), w=None) == CODES["CHAIN_ERR_DTYPE"]
    assert call(so=td([1, 2, 128, 64], chain.F32, FAKE + 5 * G), w=None) == CODES["CHAIN_ERR_SHAPE"]
    assert call(k=td([1, 3, 256, 128], chain.BF16, FAKE + G), v=td([1, 3, 256, 128], chain.BF16, FAKE + 2 * G),
                w=None) == CODES["CHAIN_ERR_SHAPE"]
    assert call(o=td([1, 4, 255, 128], chain.F32, FAKE + 3 * G), w=None) == CODES["CHAIN_ERR_SHAPE"]
    assert call(so=td([1, 2, 128, 128], chain.F32, FAKE + 3 * G + 4096), w=None) == CODES["CHAIN_ERR_ALIAS"]
    D96 = dict(q=td([1, 4, 256, 96], chain.BF16, FAKE), k=td([1, 2, 256, 96], chain.BF16, FAKE + G),
               v=td([1, 2, 256, 96], chain.BF16, FAKE + 2 * G), o=td([1, 4, 256, 96], chain.F32, FAKE + 3 * G),
               si=None, so=None, w=None)
    assert call(**D96) == CODES["CHAIN_ERR_UNSUPPORTED"]
    # zero rows with no state to pass: nothing to do
    E = dict(q=td([1, 4, 0, 128], chain.BF16, FAKE), k=td([1, 2, 0, 128], chain.BF16, FAKE + G),
             v=td([1, 2, 0, 128], chain.BF16, FAKE + 2 * G), o=td([1, 4, 0, 128], chain.F32, FAKE + 3 * G),
             si=None, so=None, w=None, n=0)
    assert call(**E) == CODES["CHAIN_OK"]


def test_mlp_noalloc_refuses_before_touching_the_device(lib):
    """Shapes whose intermediate exceeds the static scratch, and invalid
    arguments, fail validation before the call looks up any device memory."""
    P = ctypes.byref
    M, K, N = 8200, 8, 4096                  # H = 67,174,400 bytes > 64 MiB
    X = td([M, K], chain.BF16, FAKE)
    W1 = td([K, N], chain.BF16, FAKE + 2 ** 30)
    W2 = td([N, K], chain.BF16, FAKE + 2 * 2 ** 30)
    O = td([M, K], chain.BF16, FAKE + 3 * 2 ** 30)
    assert lib.chain_mlp_workspace_bytes(M, N, chain.BF16) > 64 * 2 ** 20
    assert lib.chain_mlp_fwd_noalloc(P(X), P(W1), P(W2), P(O), 0, None) == CODES["CHAIN_ERR_WORKSPACE"]
    assert b"static scratch" in lib.chain_last_error()
    Xs = td([512, 256], chain.BF16, FAKE)
    W1s = td([256, 128], chain.BF16, FAKE + 2 ** 30)
    W2s = td([128, 256], chain.BF16, FAKE + 2 * 2 ** 30)
    Os = td([512, 256], chain.BF16, FAKE + 3 * 2 ** 30)
    assert lib.chain_mlp_fwd_noalloc(P(Xs), P(W1s), P(W2s), P(Os), 7, None) == CODES["CHAIN_ERR_UNSUPPORTED"]
    W1f = td([256, 128], chain.F32, FAKE + 2 ** 30)
    assert lib.chain_mlp_fwd_noalloc(P(Xs), P(W1f), P(W2s), P(Os), 0, None) == CODES["CHAIN_ERR_DTYPE"]
    Oal = td([512, 256], chain.BF16, FAKE + 256)
    assert lib.chain_mlp_fwd_noalloc(P(Xs), P(W1s), P(W2s), P(Oal), 0, None) == CODES["CHAIN_ERR_ALIAS"]
    # an empty product is valid and touches nothing
    X0 = td([0, 256], chain.BF16, FAKE)
    O0 = td([0, 256], chain.BF16, FAKE + 3 * 2 ** 30)
    assert lib.chain_mlp_fwd_noalloc(P(X0), P(W1s), P(W2s), P(O0), 0, None) == CODES["CHAIN_OK"]
