"""Oracle for the chain O = f(A.B).C -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct CPU definition of what the
HIP path computes, in float64 with numpy.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it.  The product path (``gemm_chain_amd``) never imports, calls or links it,
and this package imports nothing from the product path: the two share no code.

Sources (cited by page and section; the text of the pages is not quoted):

* METP article, FITEE doi 10.1631/FITEE.2400602, abstract -- the core unit of
  Transformer training is two consecutive matrix products with an optional
  function between them, O = f(A.B).C.  With A = Q, B = K^T, C = V and
  f = scaled, masked row softmax this is attention; with A = X, B = W1,
  C = W2 and f = GeLU it is the MLP.
* TSP article (7minutos.es, Zyphra TSP), section "Lo que realmente significa
  plegar" -- causal attention over the full, zigzag-reordered K/V context, and
  MLP partial outputs accumulated locally shard by shard.
* LASP summary (linnk.ai), abstract -- linear attention parallelised over the
  sequence by passing an intermediate key/value state between devices; the
  right-product trick and KV-state caching.
* 2D-Attention summary (scisimple.com), sections "Introduciendo la Atencion 2D"
  (tensors chunked along the context dimension) and "Comprendiendo la
  Arquitectura de los LLMs" (MHA; GQA query heads sharing one K/V head set).

Modules:
  attention -- softmax(scale.Q.K^T + causal mask).V with per-row log-sum-exp
  attention_bwd -- its gradients dQ, dK, dV for an output gradient dO
  merge     -- combination of partial (O, LSE) results
  mlp       -- act(X.W1).W2 with erf-GeLU, tanh-GeLU, SiLU or identity, and the
               gated form (act(X.Wg) * (X.Wu)).Wd
  zigzag    -- zigzag shares and chunks of a sequence; visible-pair counts
  linear_attention -- causal linear attention with a carried key/value state (LASP)
  brute     -- element-by-element loops (math.fsum / math.exp) for tiny cases

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against brute force, closed forms or invariants.  The bf16 rounding of the
probability matrix inside a fused kernel is not modelled here (the oracle is
exact float64); that detail is covered only by the tolerance.
"""

from .attention import attention, attention_rows, visible_mask
from .attention_bwd import attention_bwd, attention_bwd_loss
from .merge import lse_merge
from .mlp import gelu_erf, gelu_tanh, silu, mlp, mlp_gated, ACTIVATIONS
from .linear_attention import linear_attention, linear_attention_chunked, linear_attention_rows
from .zigzag import (natural_chunk_positions, zigzag_chunk_positions,
                     zigzag_share_positions, visible_pairs)

__all__ = [
    "attention", "attention_rows", "visible_mask", "attention_bwd", "attention_bwd_loss", "lse_merge", "gelu_erf",
    "gelu_tanh", "silu", "mlp", "mlp_gated", "ACTIVATIONS", "natural_chunk_positions",
    "zigzag_chunk_positions", "zigzag_share_positions", "visible_pairs",
    "linear_attention", "linear_attention_chunked", "linear_attention_rows",
]
