"""Element-by-element evaluation of the same definitions for tiny inputs -- oracle
(test infrastructure).

Independent second spelling of the attention, merge and MLP definitions in the
other oracle modules (same sources), written as plain Python loops over nested
lists with exactly-rounded sums (math.fsum) and math.exp/math.log/math.erf.  It
imports nothing from them; tests use it to pin the vectorised float64 oracle.
"""

import math


def _tolist(a):
    return a.tolist() if hasattr(a, "tolist") else a


def attention(q, k, v, causal, scale, q_pos=None, k_pos=None):
    """Nested lists q[B][Hq][Sq][D], k/v[B][Hkv][Sk][D] -> (O, LSE) as nested lists."""
    q, k, v = _tolist(q), _tolist(k), _tolist(v)
    B, Hq, Sq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Sk = len(k[0]), len(k[0][0])
    qp = list(range(Sq)) if q_pos is None else [int(x) for x in q_pos]
    kp = list(range(Sk)) if k_pos is None else [int(x) for x in k_pos]
    O = [[[[0.0] * D for _ in range(Sq)] for _ in range(Hq)] for _ in range(B)]
    L = [[[-math.inf] * Sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(Sq):
                js = [j for j in range(Sk) if (not causal) or kp[j] <= qp[i]]
                if not js:
                    continue
                s = {j: scale * math.fsum(q[b][h][i][d] * k[b][g][j][d] for d in range(D))
                     for j in js}
                m = max(s.values())
                lse = m + math.log(math.fsum(math.exp(s[j] - m) for j in js))
                L[b][h][i] = lse
                for d in range(D):
                    O[b][h][i][d] = math.fsum(math.exp(s[j] - lse) * v[b][g][j][d] for j in js)
    return O, L


def merge_row(o_rows, lses):
    """One output row from C partial rows o_rows[C][D] and their LSEs lses[C]."""
    live = [c for c in range(len(lses)) if lses[c] != -math.inf]
    D = len(o_rows[0])
    if not live:
        return [0.0] * D, -math.inf
    m = max(lses[c] for c in live)
    w = {c: math.exp(lses[c] - m) for c in live}
    tot = math.fsum(w.values())
    return ([math.fsum(w[c] / tot * o_rows[c][d] for c in live) for d in range(D)],
            m + math.log(tot))


def gelu(z, form="erf"):
    if form == "silu":
        return z / (1.0 + math.exp(-z)) if z >= 0 else z * math.exp(z) / (1.0 + math.exp(z))
    if form == "erf":
        return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))
    if form == "tanh":
        return 0.5 * z * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))
    return z


def mlp(x, w1, w2, form="erf"):
    x, w1, w2 = _tolist(x), _tolist(w1), _tolist(w2)
    M, K, N, K2 = len(x), len(w1), len(w1[0]), len(w2[0])
    H = [[gelu(math.fsum(x[i][kk] * w1[kk][n] for kk in range(K)), form) for n in range(N)]
         for i in range(M)]
    return [[math.fsum(H[i][n] * w2[n][c] for n in range(N)) for c in range(K2)]
            for i in range(M)]


def mlp_gated(x, wg, wu, wd, form="silu"):
    """(act(x.wg) * (x.wu)).wd element by element with math.fsum."""
    x, wg, wu, wd = _tolist(x), _tolist(wg), _tolist(wu), _tolist(wd)
    M, K, N, K2 = len(x), len(wg), len(wg[0]), len(wd[0])
    H = [[gelu(math.fsum(x[i][kk] * wg[kk][n] for kk in range(K)), form) *
          math.fsum(x[i][kk] * wu[kk][n] for kk in range(K)) for n in range(N)] for i in range(M)]
    return [[math.fsum(H[i][n] * wd[n][c] for n in range(N)) for c in range(K2)]
            for i in range(M)]


def linear_attention(q, k, v, s_in=None):
    """Causal linear attention with a carried state, element by element:
    O[b,h,i,e] = fsum_{j<=i} (fsum_d q k) v[j,e] + fsum_d q[i,d] s_in[d,e];
    S_out[b,g,d,e] = s_in[d,e] + fsum_j k[j,d] v[j,e]."""
    q, k, v = _tolist(q), _tolist(k), _tolist(v)
    B, Hq, S, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0])
    group = Hq // Hkv
    if s_in is None:
        s_in = [[[[0.0] * D for _ in range(D)] for _ in range(Hkv)] for _ in range(B)]
    else:
        s_in = _tolist(s_in)
    o = [[[[0.0] * D for _ in range(S)] for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(S):
                sc = [math.fsum(q[b][h][i][d] * k[b][g][j][d] for d in range(D)) for j in range(i + 1)]
                for e in range(D):
                    o[b][h][i][e] = math.fsum([sc[j] * v[b][g][j][e] for j in range(i + 1)] +
                                              [q[b][h][i][d] * s_in[b][g][d][e] for d in range(D)])
    s_out = [[[[math.fsum([s_in[b][g][d][e]] + [k[b][g][j][d] * v[b][g][j][e] for j in range(S)])
                for e in range(D)] for d in range(D)] for g in range(Hkv)] for b in range(B)]
    return o, s_out
