"""The pins must catch plausible mistakes: each mutant below is a copy of the
oracle with one planted error (on the CPU, in the oracle only), and at least
one pin has to fail on it."""

import math

import numpy as np
import pytest

import importlib

import oracle

# the package re-exports functions named like some of its modules
OA = importlib.import_module("oracle.attention")
OM = importlib.import_module("oracle.merge")
OMLP = importlib.import_module("oracle.mlp")
OZ = importlib.import_module("oracle.zigzag")
from oracle import brute
import oracle_pins as P


def _attention_pins(attn):
    return [
        lambda: P.check_brute(attn, brute),
        lambda: P.check_q_zero_closed_form(attn),
        lambda: P.check_constant_v(attn),
        lambda: P.check_row0(attn),
        lambda: P.check_probabilities(attn),
        lambda: P.check_two_keys(attn),
        lambda: P.check_scale_folding(attn),
        lambda: P.check_gqa(attn),
        lambda: P.check_key_permutation(attn),
        lambda: P.check_mask_orientation(attn),
        lambda: P.check_chunk_merge(attn, oracle.lse_merge, oracle.zigzag_chunk_positions,
                                    oracle.natural_chunk_positions),
    ]


def _count_failures(pins):
    failed = 0
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed += 1
    return failed


def _rows_variant(kind):
    def attend(qr, kf, vf, qpos, kpos, causal, scale):
        s = scale * (qr @ kf.T)
        if kind == "no_scale":
            s = qr @ kf.T
        if causal:
            if kind == "strict_mask":
                vis = kpos[None, :] < qpos[:, None]
            elif kind == "reversed_mask":
                vis = kpos[None, :] >= qpos[:, None]
            elif kind == "index_mask":
                vis = np.arange(kpos.size)[None, :] <= np.arange(qpos.size)[:, None]
            else:
                vis = kpos[None, :] <= qpos[:, None]
        else:
            vis = np.ones(s.shape, bool)
        s = np.where(vis, s, -np.inf)
        o = np.zeros((qr.shape[0], vf.shape[1]))
        lse = np.full(qr.shape[0], -np.inf)
        has = vis.any(axis=1)
        if has.any():
            sh = s[has]
            m = sh.max(axis=1)
            lse_h = m + np.log(np.exp(sh - m[:, None]).sum(axis=1))
            if kind == "log2_lse":
                lse_h = lse_h / math.log(2.0)
            if kind == "unnormalised":
                p = np.exp(sh - m[:, None])
            else:
                p = np.exp(sh - lse_h[:, None])
            if kind == "pk":
                o[has] = p @ kf
            elif kind == "no_max_in_lse":
                lse_h = np.log(np.exp(sh - m[:, None]).sum(axis=1))
                o[has] = p @ vf
            else:
                o[has] = p @ vf
            lse[has] = lse_h
        return o, lse
    return attend


ROW_MUTANTS = ["no_scale", "strict_mask", "reversed_mask", "index_mask", "log2_lse",
               "unnormalised", "pk", "no_max_in_lse"]


@pytest.mark.parametrize("kind", ROW_MUTANTS)
def test_attention_mutants_caught(kind, monkeypatch):
    monkeypatch.setattr(OA, "_attend_rows", _rows_variant(kind))
    assert _count_failures(_attention_pins(OA.attention)) >= 1


def test_gqa_modulo_mapping_caught():
    def attn(q, k, v, **kw):
        Hq, Hkv = q.shape[1], k.shape[1]
        idx = [h % Hkv for h in range(Hq)]
        return oracle.attention(q, k[:, idx], v[:, idx], **kw)
    assert _count_failures(_attention_pins(attn)) >= 1


def test_transposed_score_caught():
    def attn(q, k, v, *, causal, scale, q_pos=None, k_pos=None):
        # uses K as values and V as keys
        return oracle.attention(q, v, k, causal=causal, scale=scale, q_pos=q_pos, k_pos=k_pos)
    assert _count_failures(_attention_pins(attn)) >= 1


@pytest.mark.parametrize("kind", ["unnormalised", "no_shift", "wrong_lse"])
def test_merge_mutants_caught(kind, monkeypatch):
    real = OM.lse_merge

    def bad(o_parts, lse_parts):
        o_parts = np.asarray(o_parts, float)
        lse_parts = np.asarray(lse_parts, float)
        m = lse_parts.max(axis=0)
        m_safe = np.where(np.isneginf(m), 0.0, m)
        w = np.exp(lse_parts - m_safe[None])
        tot = w.sum(axis=0)
        if kind == "unnormalised":
            return (w[..., None] * o_parts).sum(0), m_safe + np.log(tot)
        if kind == "no_shift":
            return (w[..., None] * o_parts).sum(0) / tot[..., None], np.log(tot)
        o, lse = real(o_parts, lse_parts)
        return o, lse + 0.5 * (lse_parts.shape[0] > 1)
    fails = _count_failures([
        lambda: P.check_merge_properties(bad, brute),
        lambda: P.check_chunk_merge(oracle.attention, bad, oracle.zigzag_chunk_positions,
                                    oracle.natural_chunk_positions),
    ])
    assert fails >= 1


def test_gelu_mutant_caught():
    from scipy.special import erf

    def bad(z):
        z = np.asarray(z, float)
        return 0.5 * z * (1.0 + erf(z))          # forgot the 1/sqrt(2)
    assert _count_failures([lambda: P.check_gelu(bad, oracle.gelu_tanh)]) == 1


def test_mlp_mutant_caught():
    def bad(x, w1, w2, act="gelu_erf"):
        h = OMLP.ACTIVATIONS[act](np.asarray(x, float) @ np.asarray(w1, float))
        return h @ np.asarray(w2, float) + (act != "identity") * 1e-3 * h.sum()
    assert _count_failures([lambda: P.check_mlp(bad, brute)]) == 1


def test_zigzag_mutant_caught(monkeypatch):
    def bad_pieces(S, parts, r):
        n = S // (2 * parts)
        lo = np.arange(r * n, (r + 1) * n)
        hi = np.arange((parts - 1 - r + parts) * n - n, (parts - r + parts) * n - n)  # off by a piece
        return np.concatenate([lo, hi])
    monkeypatch.setattr(OZ, "_pieces", bad_pieces)
    assert _count_failures([lambda: P.check_zigzag(OZ.zigzag_share_positions,
                                                   oracle.visible_pairs)]) == 1


def test_silu_mutants_caught():
    """sigmoid without the factor z, and a sign slip inside the exponential."""
    def no_factor(z):
        return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))

    def sign_slip(z):
        z = np.asarray(z, dtype=np.float64)
        return z / (1.0 + np.exp(z))

    for bad in (no_factor, sign_slip):
        assert _count_failures([lambda: P.check_silu(bad)]) == 1


def test_gated_mlp_mutants_caught():
    """Activation on the up product instead of the gate, a missing activation,
    and gate/up products added instead of multiplied."""
    def act_on_up(x, wg, wu, wd, act="silu"):
        return (OMLP.ACTIVATIONS[act](x @ wu) * (x @ wg)) @ wd

    def no_act(x, wg, wu, wd, act="silu"):
        return ((x @ wg) * (x @ wu)) @ wd

    def added(x, wg, wu, wd, act="silu"):
        return (OMLP.ACTIVATIONS[act](x @ wg) + (x @ wu)) @ wd

    for bad in (act_on_up, no_act, added):
        assert _count_failures([lambda: P.check_mlp_gated(bad, oracle.mlp, brute)]) == 1


def test_linear_attention_mutants_caught():
    """A strict mask, a dropped carried state, a transposed state, and a state
    that forgets S_in: each must fail a pin."""
    OL = importlib.import_module("oracle.linear_attention")

    def make(kind):
        def lin(q, k, v, s_in=None):
            q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
            B, Hq, S, D = q.shape
            Hkv = k.shape[1]
            g = Hq // Hkv
            s0 = np.zeros((B, Hkv, D, D)) if s_in is None else np.asarray(s_in, dtype=np.float64)
            mask = np.tril(np.ones((S, S)), -1 if kind == "strict" else 0)
            st = s0.transpose(0, 1, 3, 2) if kind == "transposed" else s0
            o = np.zeros_like(q)
            for b in range(B):
                for h in range(Hq):
                    o[b, h] = ((q[b, h] @ k[b, h // g].T) * mask) @ v[b, h // g]
                    if kind != "no_state":
                        o[b, h] += q[b, h] @ st[b, h // g]
            kv = np.einsum("bgjd,bgje->bgde", k, v)
            return o, (kv if kind == "forget" else s0 + kv)
        return lin

    for kind in ("strict", "no_state", "transposed", "forget"):
        bad = make(kind)
        assert _count_failures([lambda: P.check_linear_attention(bad, OL.linear_attention_chunked, brute)]) == 1, kind
