"""Pins of the float64 oracle (CPU only): brute force, closed forms, invariants."""

import oracle
from oracle import brute
import oracle_pins as P


def test_attention_matches_brute_force():
    P.check_brute(oracle.attention, brute)


def test_attention_q_zero_closed_form():
    P.check_q_zero_closed_form(oracle.attention)


def test_attention_constant_v():
    P.check_constant_v(oracle.attention)


def test_attention_causal_row0_is_v0():
    P.check_row0(oracle.attention)


def test_attention_probabilities_are_library_softmax():
    P.check_probabilities(oracle.attention)


def test_attention_two_keys_logistic():
    P.check_two_keys(oracle.attention)


def test_attention_scale_folding():
    P.check_scale_folding(oracle.attention)


def test_attention_gqa_is_repeated_mha():
    P.check_gqa(oracle.attention)


def test_attention_key_permutation():
    P.check_key_permutation(oracle.attention)


def test_attention_mask_orientation():
    P.check_mask_orientation(oracle.attention)


def test_chunked_merge_equals_whole():
    P.check_chunk_merge(oracle.attention, oracle.lse_merge,
                        oracle.zigzag_chunk_positions, oracle.natural_chunk_positions)


def test_merge_properties():
    P.check_merge_properties(oracle.lse_merge, brute)


def test_gelu_points_and_identities():
    P.check_gelu(oracle.gelu_erf, oracle.gelu_tanh)


def test_mlp():
    P.check_mlp(oracle.mlp, brute)


def test_zigzag_balance():
    P.check_zigzag(oracle.zigzag_share_positions, oracle.visible_pairs)


def test_attention_rows_matches_full():
    import numpy as np
    rng = np.random.default_rng(13)
    q, k, v = P.rand_attn(rng, 2, 4, 2, 40, 40, 8)
    o, l = oracle.attention(q, k, v, causal=True, scale=0.3)
    rows = [0, 5, 39, 17]
    ro, rl = oracle.attention_rows(q, k, v, 1, 3, rows, causal=True, scale=0.3)
    assert np.array_equal(ro, o[1, 3, rows]) and np.array_equal(rl, l[1, 3, rows])


def test_silu_closed_forms_and_identities():
    P.check_silu(oracle.silu)


def test_gated_mlp_brute_force_reductions_and_shards():
    P.check_mlp_gated(oracle.mlp_gated, oracle.mlp, brute)


def test_linear_attention_brute_chunked_state_passing_and_closed_forms():
    P.check_linear_attention(oracle.linear_attention, oracle.linear_attention_chunked, brute,
                             oracle.linear_attention_rows)
