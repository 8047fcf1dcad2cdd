"""Scaled, masked softmax attention in float64 -- oracle (test infrastructure).

Definition followed (METP abstract: O = f(A.B).C with A = Q, B = K^T, C = V and
f = row softmax of the scaled scores; TSP article, "Lo que realmente significa
plegar": the attention is causal over the full key/value context; 2D-Attention
summary, "Comprendiendo la Arquitectura de los LLMs": in GQA a group of query
heads shares one key/value head):

  for batch b, query head h, key/value head g = h // (Hq // Hkv) (contiguous
  groups), and query row i at global position p_i:
    V(i)   = { j : pi_j <= p_i }  if causal, else every key j
    s_ij   = scale * sum_d Q[b,h,i,d] * K[b,g,j,d]
    LSE_i  = log sum_{j in V(i)} exp(s_ij)        (natural log)
    O[i,:] = sum_{j in V(i)} exp(s_ij - LSE_i) * V[b,g,j,:]
  A row with an empty visible set has O = 0 and LSE = -inf.

Readings where the pages are silent: the mask compares *global* positions and
includes the diagonal (a token sees itself); LSE uses the natural log; the
scale is an argument (1/sqrt(D) in every workload here).

Inputs may be any real dtype (bf16 data must be widened to float32 first, which
is exact); everything is widened to float64 and nothing is rounded in between.
Work is blocked over query rows only, so the softmax of every row always spans
its whole visible key set.
"""

import numpy as np

_ROW_BLOCK = 256


def visible_mask(q_pos, k_pos, causal):
    """Boolean [Sq, Sk]: key j is visible to query i (global positions)."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    if not causal:
        return np.ones((q_pos.size, k_pos.size), dtype=bool)
    return k_pos[None, :] <= q_pos[:, None]


def _attend_rows(qr, kf, vf, qpos, kpos, causal, scale):
    """Rows qr [n, D] (float64) against one K/V head; returns (O [n, D], LSE [n])."""
    s = scale * (qr @ kf.T)                                  # [n, Sk]
    vis = visible_mask(qpos, kpos, causal)
    s = np.where(vis, s, -np.inf)
    n = qr.shape[0]
    o = np.zeros((n, vf.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    has = vis.any(axis=1)
    if has.any():
        sh = s[has]
        m = sh.max(axis=1)
        lse_h = m + np.log(np.exp(sh - m[:, None]).sum(axis=1))
        p = np.exp(sh - lse_h[:, None])                      # masked entries -> 0
        o[has] = p @ vf
        lse[has] = lse_h
    return o, lse


def _positions(pos, n):
    if pos is None:
        return np.arange(n, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    if pos.shape != (n,):
        raise ValueError(f"positions must have shape ({n},), got {pos.shape}")
    return pos


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("Q, K, V must be [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"shape mismatch Q{q.shape} K{k.shape} V{v.shape}")
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    return B, Hq, Sq, D, Hkv, k.shape[2]


def attention(q, k, v, *, causal, scale, q_pos=None, k_pos=None):
    """Full attention.  q [B,Hq,Sq,D], k/v [B,Hkv,Sk,D] -> (O [B,Hq,Sq,D], LSE [B,Hq,Sq]) float64."""
    B, Hq, Sq, D, Hkv, Sk = _check(q, k, v)
    qpos = _positions(q_pos, Sq)
    kpos = _positions(k_pos, Sk)
    group = Hq // Hkv
    o = np.zeros((B, Hq, Sq, D), dtype=np.float64)
    lse = np.full((B, Hq, Sq), -np.inf, dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            kf = np.asarray(k[b, g], dtype=np.float64)
            vf = np.asarray(v[b, g], dtype=np.float64)
            for h in range(g * group, (g + 1) * group):
                for r0 in range(0, Sq, _ROW_BLOCK):
                    r1 = min(Sq, r0 + _ROW_BLOCK)
                    qr = np.asarray(q[b, h, r0:r1], dtype=np.float64)
                    o[b, h, r0:r1], lse[b, h, r0:r1] = _attend_rows(
                        qr, kf, vf, qpos[r0:r1], kpos, causal, scale)
    return o, lse


def attention_rows(q, k, v, b, h, rows, *, causal, scale, q_pos=None, k_pos=None):
    """The same definition evaluated for selected query rows of one (b, h).

    Used to check outputs of workloads too large to evaluate whole.
    Returns (O [len(rows), D], LSE [len(rows)]) in float64.
    """
    B, Hq, Sq, D, Hkv, Sk = _check(q, k, v)
    qpos = _positions(q_pos, Sq)
    kpos = _positions(k_pos, Sk)
    rows = np.asarray(rows, dtype=np.int64)
    g = h // (Hq // Hkv)
    kf = np.asarray(k[b, g], dtype=np.float64)
    vf = np.asarray(v[b, g], dtype=np.float64)
    qr = np.asarray(q[b, h], dtype=np.float64)[rows]
    return _attend_rows(qr, kf, vf, qpos[rows], kpos, causal, scale)
