"""Combination of partial attention results by log-sum-exp -- oracle (test infrastructure).

Source: TSP article, "Lo que realmente significa plegar" (each device folds the
partial outputs it computes into a local accumulator as pieces arrive) and the
2D-Attention summary, "Introduciendo la Atencion 2D" (attention is computed
over chunks of the context).  The pages do not print the combination rule; the
plain reading is the exact one: if part c attended to key set S_c (disjoint
sets) and produced (O_c, LSE_c), then over the union

  M      = max_c LSE_c
  w_c    = exp(LSE_c - M)
  LSE    = M + log sum_c w_c
  O      = sum_c (w_c / sum_c' w_c') * O_c

Parts with LSE_c = -inf saw no key and carry no weight; if every part is -inf,
the result is O = 0, LSE = -inf.  Float64 throughout.
"""

import numpy as np


def lse_merge(o_parts, lse_parts):
    """o_parts [C, ..., D], lse_parts [C, ...] -> (O [..., D], LSE [...]) in float64."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    if o_parts.shape[:-1] != lse_parts.shape:
        raise ValueError(f"shape mismatch {o_parts.shape} vs {lse_parts.shape}")
    m = lse_parts.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe[None])                 # -inf parts -> weight 0
    total = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(total))
        frac = np.where(empty[None], 0.0, w / np.where(empty, 1.0, total)[None])
    o = (frac[..., None] * o_parts).sum(axis=0)
    return o, lse
