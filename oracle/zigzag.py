"""Zigzag shares and chunks of a sequence -- oracle (test infrastructure).

Source: TSP article, "Lo que realmente significa plegar": before the attention,
K and V are reordered by a zigzag partition so that causal work is balanced
across ranks (later tokens attend to longer prefixes).  The page names the
scheme but does not spell it out; the reading used here is the usual one:
cut the sequence into 2P equal pieces and give share r the pieces r and
2P-1-r, kept in ascending position order.  A sequence cut into C zigzag KV
chunks uses the same rule with P = C; natural chunks are C equal contiguous
ranges.
"""

import numpy as np


def _pieces(S, parts, r):
    if parts <= 0 or S % (2 * parts):
        raise ValueError(f"sequence {S} does not split into {2 * parts} equal pieces")
    if not 0 <= r < parts:
        raise ValueError(f"share {r} out of range [0, {parts})")
    n = S // (2 * parts)
    lo = np.arange(r * n, (r + 1) * n, dtype=np.int64)
    hi = np.arange((2 * parts - 1 - r) * n, (2 * parts - r) * n, dtype=np.int64)
    return np.concatenate([lo, hi])


def zigzag_share_positions(S, P, r):
    """Global positions held by rank r of P in a zigzag split of S tokens."""
    return _pieces(S, P, r)


def zigzag_chunk_positions(Sk, C, s):
    """Global key positions of zigzag chunk s of C."""
    return _pieces(Sk, C, s)


def natural_chunk_positions(Sk, C, s):
    """Global key positions of natural (contiguous) chunk s of C."""
    if C <= 0 or Sk % C:
        raise ValueError(f"sequence {Sk} does not split into {C} equal chunks")
    n = Sk // C
    return np.arange(s * n, (s + 1) * n, dtype=np.int64)


def visible_pairs(q_pos, k_pos):
    """Number of (query, key) pairs with key position <= query position."""
    k_sorted = np.sort(np.asarray(k_pos, dtype=np.int64))
    q = np.asarray(q_pos, dtype=np.int64)
    return int(np.searchsorted(k_sorted, q, side="right").sum())
