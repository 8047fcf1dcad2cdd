"""Pins of the float64 oracle against things other than itself.

Each ``check_*`` takes the implementation under test as an argument so that the
same checks run against the real oracle (tests/test_oracle_*.py) and against
deliberately broken copies of it (tests/test_oracle_mutants.py), which proves
that a plausible mistake -- a dropped term, a wrong sign, index or operand --
fails at least one pin.  What pins what:

  brute force      : oracle.brute (exactly rounded loops) on tiny shapes
  closed forms     : Q = 0 gives prefix means and LSE = log(i + 1); two keys
                     give a logistic mix; GeLU at table points
  special cases    : causal row 0 equals V[0]; V = identity exposes P, which must
                     equal scipy.special.softmax of the masked scores
  invariants       : constant V, scale folding, GQA = repeated MHA, key
                     permutation, mask orientation, chunk + merge = whole,
                     merge(x, x) = (O, LSE + log 2), MLP shard sum, zigzag balance
"""

import math
import os

import numpy as np
from scipy.special import softmax as sp_softmax

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_attn(rng, B, Hq, Hkv, Sq, Sk, D, amp=1.0):
    q = rng.standard_normal((B, Hq, Sq, D)) * amp
    k = rng.standard_normal((B, Hkv, Sk, D)) * amp
    v = rng.standard_normal((B, Hkv, Sk, D)) * amp
    return q, k, v


# ----------------------------------------------------------------- attention

def check_brute(attention, brute, seed=0):
    rng = np.random.default_rng(seed)
    cases = [
        (1, 1, 1, 7, 7, 4, True, None, None),
        (2, 4, 2, 9, 9, 8, True, None, None),
        (1, 4, 1, 5, 11, 3, False, None, None),
        (1, 2, 2, 6, 10, 5, True, [3, 4, 9, 12, 13, 20], list(range(0, 20, 2))),
        # rows 0 and 1 see nothing: their keys all lie later
        (1, 2, 1, 4, 5, 4, True, [0, 1, 30, 31], [5, 6, 7, 8, 29]),
    ]
    for (B, Hq, Hkv, Sq, Sk, D, causal, qp, kp) in cases:
        q, k, v = rand_attn(rng, B, Hq, Hkv, Sq, Sk, D)
        scale = 1.0 / math.sqrt(D)
        o, l = attention(q, k, v, causal=causal, scale=scale, q_pos=qp, k_pos=kp)
        ob, lb = brute.attention(q, k, v, causal, scale, qp, kp)
        ob, lb = np.array(ob), np.array(lb)
        assert np.array_equal(np.isneginf(l), np.isneginf(lb))
        fin = np.isfinite(lb)
        assert np.max(np.abs(l[fin] - lb[fin]), initial=0.0) <= 1e-12
        assert np.max(np.abs(o - ob)) <= 1e-12


def check_q_zero_closed_form(attention):
    rng = np.random.default_rng(1)
    S, D = 37, 6
    q = np.zeros((1, 1, S, D))
    _, k, v = rand_attn(rng, 1, 1, 1, S, S, D)
    o, l = attention(q, k, v, causal=True, scale=0.3)
    # all scores are 0: uniform weights over the visible prefix
    prefix_mean = np.cumsum(v[0, 0], axis=0) / np.arange(1, S + 1)[:, None]
    assert np.max(np.abs(o[0, 0] - prefix_mean)) <= 1e-13
    assert np.max(np.abs(l[0, 0] - np.log(np.arange(1, S + 1)))) <= 1e-13
    o, l = attention(q, k, v, causal=False, scale=0.3)
    assert np.max(np.abs(o[0, 0] - v[0, 0].mean(axis=0))) <= 1e-13
    assert np.max(np.abs(l[0, 0] - math.log(S))) <= 1e-13


def check_constant_v(attention):
    rng = np.random.default_rng(2)
    q, k, _ = rand_attn(rng, 1, 2, 1, 19, 19, 5)
    c = rng.standard_normal(5)
    v = np.broadcast_to(c, (1, 1, 19, 5)).copy()
    for causal in (True, False):
        o, _ = attention(q, k, v, causal=causal, scale=0.5)
        assert np.max(np.abs(o - c)) <= 1e-13


def check_row0(attention):
    rng = np.random.default_rng(3)
    q, k, v = rand_attn(rng, 1, 1, 1, 16, 16, 8)
    o, l = attention(q, k, v, causal=True, scale=0.25)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])
    assert abs(l[0, 0, 0] - 0.25 * float(q[0, 0, 0] @ k[0, 0, 0])) <= 1e-14


def check_probabilities(attention):
    """V = identity makes O the probability matrix itself."""
    rng = np.random.default_rng(4)
    S = 12
    q, k, _ = rand_attn(rng, 1, 1, 1, S, S, S)
    v = np.eye(S)[None, None]
    scale = 0.4
    for causal in (True, False):
        o, l = attention(q, k, v, causal=causal, scale=scale)
        scores = scale * np.einsum("id,jd->ij", q[0, 0], k[0, 0])
        if causal:
            scores = np.where(np.tril(np.ones((S, S), bool)), scores, -np.inf)
        ref = sp_softmax(scores, axis=1)
        assert np.max(np.abs(o[0, 0].sum(axis=1) - 1.0)) <= 1e-12
        assert np.max(np.abs(o[0, 0] - ref)) <= 1e-13
        from scipy.special import logsumexp
        assert np.max(np.abs(l[0, 0] - logsumexp(scores, axis=1))) <= 1e-12


def check_two_keys(attention):
    rng = np.random.default_rng(5)
    q, k, v = rand_attn(rng, 1, 1, 1, 3, 2, 4)
    o, l = attention(q, k, v, causal=False, scale=1.0)
    s = q[0, 0] @ k[0, 0].T                                   # [3, 2]
    w0 = 1.0 / (1.0 + np.exp(s[:, 1] - s[:, 0]))             # logistic of the difference
    ref = w0[:, None] * v[0, 0, 0] + (1.0 - w0)[:, None] * v[0, 0, 1]
    assert np.max(np.abs(o[0, 0] - ref)) <= 1e-13
    assert np.max(np.abs(l[0, 0] - np.logaddexp(s[:, 0], s[:, 1]))) <= 1e-13


def check_scale_folding(attention):
    rng = np.random.default_rng(6)
    q, k, v = rand_attn(rng, 1, 2, 2, 10, 10, 4)
    o1, l1 = attention(q, k, v, causal=True, scale=0.125)
    o2, l2 = attention(q * 0.125, k, v, causal=True, scale=1.0)
    assert np.max(np.abs(o1 - o2)) <= 1e-13
    assert np.max(np.abs(l1 - l2)) <= 1e-13
    # a different scale must change the result
    o3, _ = attention(q, k, v, causal=True, scale=0.5)
    assert np.max(np.abs(o1 - o3)) > 1e-3


def check_gqa(attention):
    rng = np.random.default_rng(7)
    q, k, v = rand_attn(rng, 2, 8, 2, 9, 9, 4)
    o, l = attention(q, k, v, causal=True, scale=0.5)
    kr = np.repeat(k, 4, axis=1)          # head h uses kv head h // 4
    vr = np.repeat(v, 4, axis=1)
    o2, l2 = attention(q, kr, vr, causal=True, scale=0.5)
    assert np.max(np.abs(o - o2)) <= 1e-14
    assert np.max(np.abs(l - l2)) <= 1e-14


def check_key_permutation(attention):
    rng = np.random.default_rng(8)
    q, k, v = rand_attn(rng, 1, 1, 1, 8, 8, 4)
    perm = rng.permutation(8)
    o1, l1 = attention(q, k, v, causal=True, scale=0.5)
    o2, l2 = attention(q, k[:, :, perm], v[:, :, perm], causal=True, scale=0.5,
                       k_pos=np.arange(8)[perm])
    assert np.max(np.abs(o1 - o2)) <= 1e-13
    assert np.max(np.abs(l1 - l2)) <= 1e-13


def check_mask_orientation(attention):
    """Row i depends on keys 0..i only, and on key i itself."""
    rng = np.random.default_rng(9)
    S = 10
    q, k, v = rand_attn(rng, 1, 1, 1, S, S, 4)
    o, l = attention(q, k, v, causal=True, scale=0.5)
    for j in range(S):
        v2 = v.copy()
        v2[0, 0, j] += 1.0
        k2 = k.copy()
        k2[0, 0, j] += 1.0
        o2, _ = attention(q, k2, v2, causal=True, scale=0.5)
        d = np.abs(o2[0, 0] - o[0, 0]).max(axis=1)
        assert np.all(d[:j] == 0.0), f"rows before {j} changed"
        assert np.all(d[j:] > 0.0), f"rows from {j} on did not change"


def check_chunk_merge(attention, lse_merge, zigzag_chunk_positions, natural_chunk_positions):
    rng = np.random.default_rng(10)
    S, D, C = 32, 4, 4
    q, k, v = rand_attn(rng, 1, 2, 1, S, S, D)
    full_o, full_l = attention(q, k, v, causal=True, scale=0.5)
    for chunker in (zigzag_chunk_positions, natural_chunk_positions):
        parts_o, parts_l = [], []
        for s in rng.permutation(C):
            pos = chunker(S, C, int(s))
            po, pl = attention(q, k[:, :, pos], v[:, :, pos], causal=True, scale=0.5, k_pos=pos)
            parts_o.append(po)
            parts_l.append(pl)
        mo, ml = lse_merge(np.stack(parts_o), np.stack(parts_l))
        assert np.max(np.abs(mo - full_o)) <= 1e-13
        assert np.max(np.abs(ml - full_l)) <= 1e-13


# --------------------------------------------------------------------- merge

def check_merge_properties(lse_merge, brute):
    rng = np.random.default_rng(11)
    o = rng.standard_normal((3, 5, 4))
    l = rng.standard_normal((3, 5)) * 3
    # one part is the identity
    mo, ml = lse_merge(o[:1], l[:1])
    assert np.max(np.abs(mo - o[0])) <= 1e-15 and np.max(np.abs(ml - l[0])) <= 1e-15
    # a part merged with itself: same O, LSE + log 2
    mo, ml = lse_merge(np.stack([o[0], o[0]]), np.stack([l[0], l[0]]))
    assert np.max(np.abs(mo - o[0])) <= 1e-15
    assert np.max(np.abs(ml - (l[0] + math.log(2.0)))) <= 1e-14
    # -inf parts carry no weight; all -inf gives (0, -inf), never NaN
    l2 = l.copy()
    l2[1, :] = -np.inf
    mo, ml = lse_merge(o, l2)
    mo_ref, ml_ref = lse_merge(o[[0, 2]], l[[0, 2]])
    assert np.max(np.abs(mo - mo_ref)) <= 1e-14 and np.max(np.abs(ml - ml_ref)) <= 1e-14
    l3 = np.full_like(l, -np.inf)
    mo, ml = lse_merge(o, l3)
    assert np.all(mo == 0.0) and np.all(np.isneginf(ml)) and not np.isnan(mo).any()
    # element-wise brute force
    mo, ml = lse_merge(o, l2)
    for r in range(5):
        bo, bl = brute.merge_row(o[:, r].tolist(), l2[:, r].tolist())
        assert np.max(np.abs(mo[r] - np.array(bo))) <= 1e-14 and abs(ml[r] - bl) <= 1e-14


# ----------------------------------------------------------------------- MLP

def load_gelu_points():
    pts = []
    with open(os.path.join(GOLDEN, "gelu_points.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                x, y = line.split()
                pts.append((float(x), float(y)))
    return pts


def check_gelu(gelu_erf, gelu_tanh):
    for x, y in load_gelu_points():
        assert abs(float(gelu_erf(x)) - y) <= 2e-16 * max(1.0, abs(y)) * 4
    xs = np.linspace(-6, 6, 2001)
    # x*Phi(x) - (-x)*Phi(-x) = x
    assert np.max(np.abs(gelu_erf(xs) - gelu_erf(-xs) - xs)) <= 1e-14
    # tanh approximation stays within 5e-4 of the exact form
    assert np.max(np.abs(gelu_tanh(xs) - gelu_erf(xs))) <= 5e-4
    assert np.max(np.abs(gelu_tanh(xs) - gelu_erf(xs))) >= 1e-5


def check_mlp(mlp, brute):
    rng = np.random.default_rng(12)
    M, K, N, K2 = 7, 6, 5, 4
    x = rng.standard_normal((M, K))
    w1 = rng.standard_normal((K, N)) * 0.5
    w2 = rng.standard_normal((N, K2)) * 0.5
    for act, form in (("gelu_erf", "erf"), ("gelu_tanh", "tanh"), ("identity", "id")):
        o = mlp(x, w1, w2, act)
        ob = np.array(brute.mlp(x, w1, w2, form))
        assert np.max(np.abs(o - ob)) <= 1e-13
    assert np.all(mlp(np.zeros((M, K)), w1, w2, "gelu_erf") == 0.0)
    assert np.max(np.abs(mlp(x, w1, w2, "identity") - x @ (w1 @ w2))) <= 1e-13
    # shards of the inner dimension summed locally give the whole product
    full = mlp(x, w1, w2, "gelu_erf")
    parts = sum(mlp(x, w1[:, s:s + 2], w2[s:s + 2], "gelu_erf") for s in range(0, N, 2))
    assert np.max(np.abs(parts - full)) <= 1e-13


def check_silu(silu):
    ln3 = math.log(3.0)
    # sigmoid(ln 3) = 3/4
    assert abs(float(silu(ln3)) - 0.75 * ln3) <= 1e-16 * 4
    assert float(silu(0.0)) == 0.0
    xs = np.linspace(-30.0, 30.0, 601)
    # z*s(z) - (-z)*s(-z) = z (s(z) + s(-z) = 1)
    assert np.max(np.abs(silu(xs) - silu(-xs) - xs)) <= 1e-13
    # far tails: z for large z, z*e^z for very negative z
    assert abs(float(silu(40.0)) - 40.0) <= 40.0 * 1e-15
    assert abs(float(silu(-40.0)) - (-40.0 * math.exp(-40.0))) <= 1e-30
    # z/2 + z^2/4 + O(z^4) at the origin
    assert abs(float(silu(1e-8)) - (0.5e-8 + 0.25e-16)) <= 1e-23


def check_mlp_gated(mlp_gated, mlp, brute):
    rng = np.random.default_rng(13)
    M, K, N, K2 = 6, 5, 4, 3
    x = rng.standard_normal((M, K))
    wg = rng.standard_normal((K, N)) * 0.5
    wu = rng.standard_normal((K, N)) * 0.5
    wd = rng.standard_normal((N, K2)) * 0.5
    for act, form in (("silu", "silu"), ("gelu_erf", "erf"), ("identity", "id")):
        o = mlp_gated(x, wg, wu, wd, act)
        ob = np.array(brute.mlp_gated(x, wg, wu, wd, form))
        assert np.max(np.abs(o - ob)) <= 1e-13
    # up product identically 1 (a column of ones in X, selected by Wu): the plain chain
    x1 = x.copy()
    x1[:, 0] = 1.0
    w_one = np.zeros((K, N))
    w_one[0, :] = 1.0
    for act in ("silu", "gelu_erf"):
        assert np.max(np.abs(mlp_gated(x1, wg, w_one, wd, act) - mlp(x1, wg, wd, act))) <= 1e-13
    # the activation acts on the gate product only: with the gate product identically 1,
    # the result is act(1) times the plain linear chain through Wu
    for act, a1 in (("silu", 1.0 / (1.0 + math.exp(-1.0))), ("identity", 1.0)):
        ref = a1 * (x1 @ wu) @ wd
        assert np.max(np.abs(mlp_gated(x1, w_one, wu, wd, act) - ref)) <= 1e-13
    # identity activation: gate and up are interchangeable
    assert np.max(np.abs(mlp_gated(x, wg, wu, wd, "identity") - mlp_gated(x, wu, wg, wd, "identity"))) <= 1e-13
    assert np.all(mlp_gated(np.zeros((M, K)), wg, wu, wd, "silu") == 0.0)
    # shards of the inner dimension (gate, up and down together) sum to the whole
    full = mlp_gated(x, wg, wu, wd, "silu")
    parts = sum(mlp_gated(x, wg[:, s:s + 2], wu[:, s:s + 2], wd[s:s + 2], "silu") for s in range(0, N, 2))
    assert np.max(np.abs(parts - full)) <= 1e-13


# --------------------------------------------------------- linear attention

def check_linear_attention(lin, lin_chunked, brute, lin_rows=None):
    OLR = lin_rows if lin_rows is not None else (lambda q, k, v, rows, s: lin(q, k, v, s)[0][:, :, rows])
    rng = np.random.default_rng(21)
    # brute force on tiny shapes, GQA 2:1, with a carried state
    q = rng.standard_normal((1, 2, 5, 3))
    k = rng.standard_normal((1, 1, 5, 3))
    v = rng.standard_normal((1, 1, 5, 3))
    s_in = rng.standard_normal((1, 1, 3, 3))
    o, so = lin(q, k, v, s_in)
    ob, sob = brute.linear_attention(q, k, v, s_in)
    assert np.max(np.abs(o - np.array(ob))) <= 1e-13
    assert np.max(np.abs(so - np.array(sob))) <= 1e-13
    # the right-product chunk recurrence equals the definition (ragged last chunk)
    q = rng.standard_normal((2, 4, 37, 8))
    k = rng.standard_normal((2, 2, 37, 8))
    v = rng.standard_normal((2, 2, 37, 8))
    s_in = rng.standard_normal((2, 2, 8, 8))
    o, so = lin(q, k, v, s_in)
    for chunk in (1, 5, 16, 37, 64):
        oc, soc = lin_chunked(q, k, v, chunk, s_in)
        assert np.max(np.abs(oc - o)) <= 1e-11 and np.max(np.abs(soc - so)) <= 1e-11
    # state passing: the second share with the first share's state continues the sequence
    o1, s1 = lin(q[:, :, :20], k[:, :, :20], v[:, :, :20], s_in)
    o2, s2 = lin(q[:, :, 20:], k[:, :, 20:], v[:, :, 20:], s1)
    assert np.max(np.abs(np.concatenate([o1, o2], axis=2) - o)) <= 1e-11
    assert np.max(np.abs(s2 - so)) <= 1e-11
    # closed forms: V = 1 gives every column q_i . sum_{j<=i} k_j; K = 0 gives Q S_in
    ones = np.ones_like(v)
    o, _ = lin(q, k, ones)
    pref = np.cumsum(np.repeat(k, 2, axis=1), axis=2)
    expect = np.einsum("bhid,bhid->bhi", q, pref)
    assert np.max(np.abs(o - expect[..., None])) <= 1e-11
    o, so = lin(q, np.zeros_like(k), v, s_in)
    assert np.max(np.abs(o - np.einsum("bhid,bhde->bhie", q, np.repeat(s_in, 2, axis=1)))) <= 1e-12
    assert np.array_equal(so, s_in)
    # selected rows by the definition agree with the full evaluation
    rows = [0, 5, 36]
    o_full, _ = lin(q, k, v, s_in)
    assert np.max(np.abs(OLR(q, k, v, rows, s_in) - o_full[:, :, rows])) <= 1e-11
    # row 0 sees only key 0: O_0 = (q_0 . k_0) v_0 without a state
    o, _ = lin(q, k, v)
    r0 = np.einsum("bhd,bhd->bh", q[:, :, 0], np.repeat(k[:, :, 0], 2, axis=1))[..., None] * np.repeat(v[:, :, 0], 2, axis=1)
    assert np.max(np.abs(o[:, :, 0] - r0)) <= 1e-12


# -------------------------------------------------------------------- zigzag

def check_zigzag(zigzag_share_positions, visible_pairs):
    for P, n in ((1, 3), (2, 5), (4, 4), (8, 16)):
        S = 2 * P * n
        shares = [zigzag_share_positions(S, P, r) for r in range(P)]
        allpos = np.sort(np.concatenate(shares))
        assert np.array_equal(allpos, np.arange(S))
        for r, pos in enumerate(shares):
            assert np.all(np.diff(pos) > 0)
            assert pos[0] == r * n and pos[-1] == (2 * P - r) * n - 1
            # brute count of causal pairs of this share against the whole context
            brute = sum(1 for p in pos.tolist() for kpos in range(S) if kpos <= p)
            assert visible_pairs(pos, np.arange(S)) == brute
            # balanced work: every share sees 2*P*n^2 + n pairs
            assert brute == 2 * P * n * n + n
