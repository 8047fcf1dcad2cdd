"""Causal linear attention with a carried key/value state, in float64 -- oracle
(test infrastructure).

Source: the LASP summary (linnk.ai, "Effiziente Parallelisierung linearer
Aufmerksamkeitssequenzen"), abstract: linear attention is parallelised over the
sequence by passing an intermediate state from device to device in the forward
and backward passes; the right-product trick of linear attention, kernel fusion
and caching of the intermediate KV state make it fast.  It is the chain
O = f(A.B).C of the METP abstract with A = Q, B = K^T, C = V and f the causal
mask alone (no softmax).

Readings where the page is silent (it prints no formula): no normalisation and
no decay, so for batch b, query head h and its key/value head g = h // (Hq // Hkv)

  O[i, :]   = sum_{j <= i} (Q[b,h,i,:] . K[b,g,j,:]) V[b,g,j,:]  +  Q[b,h,i,:] S_in[b,g]
  S_out[b,g] = S_in[b,g] + sum_j K[b,g,j,:]^T V[b,g,j,:]          (a D x D matrix, D_k x D_v)

S_in is the state a previous device hands over (zero for the first share of a
sequence).  This module writes the left-product definition above literally
(an S x S masked score matrix per head); the right-product, chunked evaluation
is what the kernels do and what the pins compare against.

Inputs of any real dtype are widened to float64; nothing is rounded.
"""

import numpy as np


def _widen(*xs):
    return [np.asarray(x, dtype=np.float64) for x in xs]


def linear_attention(q, k, v, s_in=None):
    """(O [B,Hq,S,D], S_out [B,Hkv,D,D]) in float64 from q [B,Hq,S,D], k, v
    [B,Hkv,S,D] and an optional carried state s_in [B,Hkv,D,D] (zero if None)."""
    q, k, v = _widen(q, k, v)
    B, Hq, S, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != S or k.shape[3] != D:
        raise ValueError(f"K/V shape {k.shape} does not match Q {q.shape}")
    Hkv = k.shape[1]
    if Hkv == 0 or Hq % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    group = Hq // Hkv
    s_in = np.zeros((B, Hkv, D, D)) if s_in is None else np.asarray(s_in, dtype=np.float64)
    mask = np.tril(np.ones((S, S)))
    o = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            scores = (q[b, h] @ k[b, g].T) * mask
            o[b, h] = scores @ v[b, g] + q[b, h] @ s_in[b, g]
    s_out = s_in + np.einsum("bgjd,bgje->bgde", k, v)
    return o, s_out


def linear_attention_chunked(q, k, v, chunk, s_in=None):
    """The same result by the right-product recurrence over chunks of `chunk`
    rows: O_t = mask(Q_t K_t^T) V_t + Q_t S_{t-1}, S_t = S_{t-1} + K_t^T V_t.
    Test infrastructure for the pins (the kernels' evaluation order)."""
    q, k, v = _widen(q, k, v)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    state = np.zeros((B, Hkv, D, D)) if s_in is None else np.array(s_in, dtype=np.float64)
    o = np.zeros_like(q)
    for t0 in range(0, S, chunk):
        t1 = min(t0 + chunk, S)
        m = np.tril(np.ones((t1 - t0, t1 - t0)))
        for b in range(B):
            for h in range(Hq):
                g = h // group
                qt, kt, vt = q[b, h, t0:t1], k[b, g, t0:t1], v[b, g, t0:t1]
                o[b, h, t0:t1] = ((qt @ kt.T) * m) @ vt + qt @ state[b, g]
        state = state + np.einsum("bgjd,bgje->bgde", k[:, :, t0:t1], v[:, :, t0:t1])
    return o, state


def linear_attention_rows(q, k, v, rows, s_in=None):
    """O at the given query rows only, by the definition (each row against its
    key prefix): [B, Hq, len(rows), D] in float64.  For checks at sizes where the
    full S x S score matrix does not fit."""
    q, k, v = _widen(q, k, v)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    s_in = np.zeros((B, Hkv, D, D)) if s_in is None else np.asarray(s_in, dtype=np.float64)
    out = np.zeros((B, Hq, len(rows), D))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for n, i in enumerate(rows):
                sc = k[b, g, :i + 1] @ q[b, h, i]
                out[b, h, n] = sc @ v[b, g, :i + 1] + q[b, h, i] @ s_in[b, g]
    return out
