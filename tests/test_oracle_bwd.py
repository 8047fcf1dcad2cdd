"""Pins of the attention-gradient oracle (CPU): finite differences of the forward
oracle, closed forms and the GQA reduction."""

import numpy as np
import pytest

import oracle


def _inputs(B, Hq, Hkv, S, D, seed):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, S, D))
    k = r.standard_normal((B, Hkv, S, D))
    v = r.standard_normal((B, Hkv, S, D))
    do = r.standard_normal((B, Hq, S, D))
    return q, k, v, do


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2)])
def test_gradients_match_central_differences(causal, Hq, Hkv):
    """d/dx sum(O * dO) by central differences of the forward oracle, for every
    entry of Q, K and V: an independent check of every term of the backward."""
    q, k, v, do = _inputs(1, Hq, Hkv, 5, 3, 7 + Hq)
    scale = 0.7
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=causal, scale=scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}; args_p[name] = xp
            args_m = {"q": q, "k": k, "v": v}; args_m[name] = xm
            lp = oracle.attention_bwd_loss(args_p["q"], args_p["k"], args_p["v"], do, causal, scale)
            lm = oracle.attention_bwd_loss(args_m["q"], args_m["k"], args_m["v"], do, causal, scale)
            num[idx] = (lp - lm) / (2 * h)
        assert np.abs(num - g).max() < 1e-7, (name, np.abs(num - g).max())


def test_constant_values_give_zero_query_and_key_gradients():
    """V equal on every key: O is that row, dP is constant along each row, so
    dS = 0 (dQ = dK = 0) and dV = P^T dO."""
    q, k, _, do = _inputs(1, 2, 2, 9, 4, 3)
    row = np.array([0.5, -1.0, 2.0, 0.25])
    v = np.broadcast_to(row, (1, 2, 9, 4)).copy()
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=True, scale=0.5)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    # column sums of P^T dO: sum over keys of dV equals sum over queries of dO
    assert np.allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)


def test_gqa_equals_repeated_heads_with_summed_key_value_gradients():
    q, k, v, do = _inputs(2, 4, 2, 7, 5, 11)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=True, scale=0.4)
    kr = np.repeat(k, 2, axis=1)
    vr = np.repeat(v, 2, axis=1)
    dq2, dk2, dv2 = oracle.attention_bwd(q, kr, vr, do, causal=True, scale=0.4)
    assert np.allclose(dq, dq2, atol=1e-13)
    assert np.allclose(dk, dk2.reshape(2, 2, 2, 7, 5).sum(axis=2), atol=1e-13)
    assert np.allclose(dv, dv2.reshape(2, 2, 2, 7, 5).sum(axis=2), atol=1e-13)


def test_first_causal_row_sees_only_itself():
    """Row 0 of causal attention attends to key 0 alone (P = 1): its dQ is zero
    (dS = 1 * (dP - dP) = 0) and it adds dO[0] to dV[0]."""
    q, k, v, do = _inputs(1, 1, 1, 4, 3, 5)
    do2 = do.copy(); do2[:, :, 1:] = 0.0
    dq, dk, dv = oracle.attention_bwd(q, k, v, do2, causal=True, scale=1.0)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    assert np.allclose(dv[0, 0, 0], do2[0, 0, 0]) and np.abs(dv[0, 0, 1:]).max() < 1e-14


def test_a_dropped_row_term_fails_the_difference_pin():
    """The plausible mistake D_i = 0 (dS = P * dP) is rejected by the
    central-difference comparison that the oracle passes."""
    q, k, v, do = _inputs(1, 1, 1, 4, 3, 9)
    good = oracle.attention_bwd(q, k, v, do, causal=True, scale=0.8)[0]
    # recompute dQ without the D_i term, directly from the definition
    s = 0.8 * (q[0, 0] @ k[0, 0].T)
    s = np.where(np.tri(4, dtype=bool), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True)); p /= p.sum(axis=1, keepdims=True)
    dp = do[0, 0] @ v[0, 0].T
    bad = 0.8 * ((p * dp) @ k[0, 0])
    h = 1e-6
    num = np.zeros_like(q[0, 0])
    for idx in np.ndindex(num.shape):
        xp = q.copy(); xp[(0, 0) + idx] += h
        xm = q.copy(); xm[(0, 0) + idx] -= h
        num[idx] = (oracle.attention_bwd_loss(xp, k, v, do, True, 0.8) -
                    oracle.attention_bwd_loss(xm, k, v, do, True, 0.8)) / (2 * h)
    assert np.abs(num - good[0, 0]).max() < 1e-7
    assert np.abs(num - bad).max() > 1e-3
