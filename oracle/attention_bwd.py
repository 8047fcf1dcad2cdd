"""Gradients of scaled, masked softmax attention in float64 -- oracle (test infrastructure).

What is differentiated: the attention of ``oracle.attention`` (METP article,
abstract: the chain O = f(A.B).C with A = Q, B = K^T, C = V and f the scaled,
masked row softmax), as it appears in training.  The pages train these models:
the METP abstract treats the chain as the core unit of Transformer training,
the 2D-Attention summary ("Estrategias de Entrenamiento Distribuido") keeps
only what is needed and recomputes the rest in the backward pass, and the LASP
summary (abstract) runs forward and backward passes over sequence chunks.  The
pages give no formula for the backward; it is the chain rule applied to the
forward definition, written out here for an output gradient dO:

  for batch b, query head h and its key/value head g = h // (Hq // Hkv):
    P_ij   = exp(s_ij - LSE_i) on the visible set of row i, 0 elsewhere
    dV[g] += P^T dO[h]                       (summed over the group's heads)
    dP     = dO[h] V[g]^T
    D_i    = sum_j P_ij dP_ij                (equals sum_d dO[h]_id O[h]_id)
    dS_ij  = P_ij (dP_ij - D_i)
    dQ[h]  = scale * dS K[g]
    dK[g] += scale * dS^T Q[h]               (summed over the group's heads)
  A row with no visible key contributes nothing (its dQ row is 0).

Reading where the pages are silent: the gradient is taken of exactly the
forward the oracle defines (same mask, scale and GQA grouping); P is recomputed
from the scores and the log-sum-exp rather than stored.

Inputs of any real dtype are widened to float64; nothing is rounded in between.
Work is blocked over query rows; every row's softmax spans its whole visible
key set.
"""

import numpy as np

from .attention import visible_mask, _check, _positions

_ROW_BLOCK = 256


def attention_bwd(q, k, v, do, causal=True, scale=None, q_pos=None, k_pos=None):
    """(dQ [B,Hq,Sq,D], dK [B,Hkv,Sk,D], dV [B,Hkv,Sk,D]) in float64.

    q [B,Hq,Sq,D], k and v [B,Hkv,Sk,D], do [B,Hq,Sq,D]; positions as in
    ``oracle.attention`` (natural order when None).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Sq, D, Hkv, Sk = _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError(f"dO must have the shape of Q {q.shape}, got {do.shape}")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    qpos = _positions(q_pos, Sq)
    kpos = _positions(k_pos, Sk)
    group = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            kf, vf = k[b, g], v[b, g]
            for r0 in range(0, Sq, _ROW_BLOCK):
                r1 = min(r0 + _ROW_BLOCK, Sq)
                vis = visible_mask(qpos[r0:r1], kpos, causal)
                s = np.where(vis, scale * (q[b, h, r0:r1] @ kf.T), -np.inf)
                has = vis.any(axis=1)
                p = np.zeros_like(s)
                if has.any():
                    sh = s[has]
                    m = sh.max(axis=1)
                    lse = m + np.log(np.exp(sh - m[:, None]).sum(axis=1))
                    p[has] = np.exp(sh - lse[:, None])
                dor = do[b, h, r0:r1]
                dv[b, g] += p.T @ dor
                dp = dor @ vf.T
                d_row = (p * dp).sum(axis=1)
                ds = p * (dp - d_row[:, None])
                dq[b, h, r0:r1] = scale * (ds @ kf)
                dk[b, g] += scale * (ds.T @ q[b, h, r0:r1])
    return dq, dk, dv


def attention_bwd_loss(q, k, v, do, causal=True, scale=None):
    """The scalar sum(O * dO) whose gradient attention_bwd returns (for finite
    differences): O from ``oracle.attention``."""
    from .attention import attention
    if scale is None:
        scale = 1.0 / np.sqrt(np.shape(q)[3])
    o, _ = attention(q, k, v, causal=causal, scale=scale)
    return float((np.asarray(o, dtype=np.float64) * np.asarray(do, dtype=np.float64)).sum())
