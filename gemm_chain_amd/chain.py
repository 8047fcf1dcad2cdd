"""ctypes binding of libchain (include/chain.h) -- argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module
turns torch tensors into ``chain_tensor`` descriptors, allocates outputs with
torch (device memory is torch's), passes torch's current HIP stream, and turns
a non-OK status into ``ChainError``.  There is no fallback: if libchain.so is
missing or a call fails, it raises.
"""

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None

MAX_DIMS = 5
MAX_RUNS = 4

F32, BF16 = 0, 1
_DT = {torch.float32: F32, torch.bfloat16: BF16}
ACTS = {"gelu_erf": 0, "gelu_tanh": 1, "identity": 2, "silu": 3}

STATUS = ["CHAIN_OK", "CHAIN_ERR_NULL", "CHAIN_ERR_DTYPE", "CHAIN_ERR_SHAPE", "CHAIN_ERR_LAYOUT",
          "CHAIN_ERR_ALIGN", "CHAIN_ERR_ALIAS", "CHAIN_ERR_UNSUPPORTED", "CHAIN_ERR_WORKSPACE",
          "CHAIN_ERR_HIP"]


class ChainTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * MAX_DIMS), ("stride", ctypes.c_int64 * MAX_DIMS)]


class ChainSegs(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("start", ctypes.c_int64 * MAX_RUNS),
                ("len", ctypes.c_int64 * MAX_RUNS)]


class ChainError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        self.name = STATUS[status] if 0 <= status < len(STATUS) else str(status)
        super().__init__(f"{self.name}: {message}")


def library_path():
    return os.environ.get("CHAIN_LIBRARY", os.path.join(_PKG, "libchain.so"))


def load():
    """Load libchain.so once; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m gemm_chain_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    T, S = P(ChainTensor), P(ChainSegs)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sigs = {
        "chain_version": (ctypes.c_int, []),
        "chain_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "chain_last_error": (ctypes.c_char_p, []),
        "chain_attn_fwd": (ctypes.c_int, [T, T, T, T, T, ctypes.c_int, f32, ctypes.c_int, ctypes.c_int, vp]),
        "chain_attn_partial": (ctypes.c_int, [T, T, T, T, T, ctypes.c_int, f32, S, S, vp]),
        "chain_lse_merge": (ctypes.c_int, [T, T, T, T, vp]),
        "chain_mlp_fwd": (ctypes.c_int, [T, T, T, T, ctypes.c_int, vp, sz, vp]),
        "chain_mlp_workspace_bytes": (sz, [i64, i64, i32]),
        "chain_mlp_fwd_noalloc": (ctypes.c_int, [T, T, T, T, ctypes.c_int, vp]),
        "chain_mlp_gated_fwd": (ctypes.c_int, [T, T, T, T, T, ctypes.c_int, vp, sz, vp]),
        "chain_attn_bwd": (ctypes.c_int, [T, T, T, T, T, T, T, T, T, ctypes.c_int, f32, vp, sz, vp]),
        "chain_attn_bwd_workspace_bytes": (sz, [i64, i64, i64]),
        "chain_linear_attn_fwd": (ctypes.c_int, [T, T, T, T, T, T, vp, sz, vp]),
        "chain_linear_attn_workspace_bytes": (sz, [i64, i64, i64, i64]),
        "chain_zigzag_segs": (ctypes.c_int, [i64, i32, i32, S]),
        "chain_attn_tile_census": (ctypes.c_int, [i64, S, i64, S, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                  P(i64), P(i64), P(i64)]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _check(status):
    if status != 0:
        raise ChainError(status, load().chain_last_error().decode())


def desc(t):
    """chain_tensor describing torch tensor t (no copy)."""
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() > MAX_DIMS:
        raise ValueError("too many dimensions")
    d = ChainTensor()
    d.data = t.data_ptr() if t.numel() else None
    d.dtype = _DT[t.dtype]
    d.ndim = t.dim()
    for i, (n, s) in enumerate(zip(t.shape, t.stride())):
        d.shape[i] = n
        d.stride[i] = s
    return d


def segs(runs):
    """chain_segs from a list of (start, length) runs."""
    if isinstance(runs, ChainSegs):
        return runs
    s = ChainSegs()
    runs = list(runs)
    if not 1 <= len(runs) <= MAX_RUNS:
        raise ValueError(f"1..{MAX_RUNS} runs expected")
    s.n = len(runs)
    for i, (a, n) in enumerate(runs):
        s.start[i] = int(a)
        s.len[i] = int(n)
    return s


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _scale(scale, D):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def attn_fwd(q, k, v, causal=True, scale=None, n_chunks=1, zigzag=False, out=None, lse=None):
    """Whole attention with chunked online-softmax merge; returns (O, LSE)."""
    lib = load()
    B, Hq, S, D = q.shape
    o = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    l = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(lib.chain_attn_fwd(desc(q), desc(k), desc(v), desc(o), desc(l), int(bool(causal)),
                              _scale(scale, D), int(n_chunks), int(bool(zigzag)), _stream(q)))
    return o, l


def attn_partial(q, kc, vc, q_pos, kv_pos, causal=True, scale=None, out=None, lse=None):
    """One ring step: f32 partial (O_part, LSE_part) of q against one key/value chunk."""
    lib = load()
    B, Hq, S, D = q.shape
    o = torch.empty((B, Hq, S, D), dtype=torch.float32, device=q.device) if out is None else out
    l = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device) if lse is None else lse
    qs, ks = segs(q_pos), segs(kv_pos)
    _check(lib.chain_attn_partial(desc(q), desc(kc), desc(vc), desc(o), desc(l), int(bool(causal)),
                                  _scale(scale, D), ctypes.byref(qs), ctypes.byref(ks), _stream(q)))
    return o, l


def lse_merge(o_parts, lse_parts, out_dtype=torch.bfloat16, out=None, lse=None, want_lse=True):
    """Merge C partials [C,B,H,S,D] / [C,B,H,S] into (O, LSE)."""
    lib = load()
    C, B, H, S, D = o_parts.shape
    o = torch.empty((B, H, S, D), dtype=out_dtype, device=o_parts.device) if out is None else out
    l = lse
    if l is None and want_lse:
        l = torch.empty((B, H, S), dtype=torch.float32, device=o_parts.device)
    _check(lib.chain_lse_merge(desc(o_parts), desc(lse_parts), desc(o),
                               desc(l) if l is not None else None, _stream(o_parts)))
    return o, l


def attn_bwd_workspace_bytes(B, Hq, S):
    return int(load().chain_attn_bwd_workspace_bytes(int(B), int(Hq), int(S)))


def attn_bwd(q, k, v, o, lse, do, causal=True, scale=None, dq=None, dk=None, dv=None,
             workspace=None):
    """(dQ, dK, dV) in f32 for bf16 attention whose forward gave (O, LSE)."""
    lib = load()
    B, Hq, S, D = q.shape
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device) if dv is None else dv
    need = attn_bwd_workspace_bytes(B, Hq, S)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib.chain_attn_bwd(desc(q), desc(k), desc(v), desc(o), desc(lse), desc(do), desc(dq),
                              desc(dk), desc(dv), int(bool(causal)), _scale(scale, D),
                              ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                              _stream(q)))
    return dq, dk, dv


def linear_attn_workspace_bytes(B, Hkv, S, D):
    return int(load().chain_linear_attn_workspace_bytes(int(B), int(Hkv), int(S), int(D)))


def linear_attn_fwd(q, k, v, s_in=None, want_state=True, out=None, out_dtype=torch.float32,
                    s_out=None, workspace=None):
    """(O, S_out) of causal linear attention carrying the state s_in (None: zero)."""
    lib = load()
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    o = torch.empty((B, Hq, S, D), dtype=out_dtype, device=q.device) if out is None else out
    so = s_out
    if so is None and want_state:
        so = torch.empty((B, Hkv, D, D), dtype=torch.float32, device=q.device)
    need = linear_attn_workspace_bytes(B, Hkv, S, D)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib.chain_linear_attn_fwd(desc(q), desc(k), desc(v), desc(o),
                                     desc(s_in) if s_in is not None else None,
                                     desc(so) if so is not None else None,
                                     ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(q)))
    return o, so


def mlp_workspace_bytes(M, N, dtype=torch.bfloat16):
    return int(load().chain_mlp_workspace_bytes(int(M), int(N), _DT[dtype]))


def mlp_fwd(x, w1, w2, act="gelu_erf", out=None, out_dtype=None, workspace=None):
    """O = act(X.W1).W2; the intermediate lives in `workspace` (allocated if None)."""
    lib = load()
    M, N, K2 = x.shape[0], w1.shape[1], w2.shape[1]
    o = torch.empty((M, K2), dtype=out_dtype or x.dtype, device=x.device) if out is None else out
    need = mlp_workspace_bytes(M, N, x.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _check(lib.chain_mlp_fwd(desc(x), desc(w1), desc(w2), desc(o), ACTS[act],
                             ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(x)))
    return o


def mlp_fwd_noalloc(x, w1, w2, act="gelu_erf", out=None, out_dtype=None):
    """O = act(X.W1).W2 with the intermediate in the library's static device scratch
    (no workspace; the library allocates nothing)."""
    lib = load()
    M, K2 = x.shape[0], w2.shape[1]
    o = torch.empty((M, K2), dtype=out_dtype or x.dtype, device=x.device) if out is None else out
    _check(lib.chain_mlp_fwd_noalloc(desc(x), desc(w1), desc(w2), desc(o), ACTS[act], _stream(x)))
    return o


def mlp_gated_fwd(x, wg, wu, wd, act="silu", out=None, out_dtype=None, workspace=None):
    """O = (act(X.Wg) * (X.Wu)).Wd; Wg and Wu column-major [K, N] views."""
    lib = load()
    M, N, K2 = x.shape[0], wg.shape[1], wd.shape[1]
    o = torch.empty((M, K2), dtype=out_dtype or x.dtype, device=x.device) if out is None else out
    need = mlp_workspace_bytes(M, N, x.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _check(lib.chain_mlp_gated_fwd(desc(x), desc(wg), desc(wu), desc(wd), desc(o), ACTS[act],
                                   ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(x)))
    return o


def zigzag_segments(S, parts, r):
    """[(start, length), (start, length)]: share r of `parts` in a zigzag split of S."""
    s = ChainSegs()
    _check(load().chain_zigzag_segs(int(S), int(parts), int(r), ctypes.byref(s)))
    return [(s.start[i], s.len[i]) for i in range(s.n)]


def tile_census(Sq, Sk, q_pos=None, kv_pos=None, n_chunks=1, zigzag=False, causal=True,
                block_m=32, block_n=64):
    """(full, diag, skip) counts of the kernels' causal tile schedule (host only)."""
    f, d, k = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    qs = ctypes.byref(segs(q_pos)) if q_pos is not None else None
    ks = ctypes.byref(segs(kv_pos)) if kv_pos is not None else None
    _check(load().chain_attn_tile_census(int(Sq), qs, int(Sk), ks, int(n_chunks), int(bool(zigzag)),
                                         int(bool(causal)), int(block_m), int(block_n),
                                         ctypes.byref(f), ctypes.byref(d), ctypes.byref(k)))
    return f.value, d.value, k.value
