"""gemm_chain_amd -- the chain O = f(A.B).C on MI355X (gfx950).

The compute lives in ``libchain.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/chain.h``).  ``gemm_chain_amd.chain`` is the thin ctypes
binding; importing this package does not load the library, the first call
does, and it raises if the library is missing.
"""

from .chain import (ChainError, attn_bwd, attn_bwd_workspace_bytes, attn_fwd, attn_partial,
                    library_path, linear_attn_fwd, linear_attn_workspace_bytes, load, lse_merge,
                    mlp_fwd, mlp_fwd_noalloc, mlp_gated_fwd, mlp_workspace_bytes, tile_census,
                    zigzag_segments)

__all__ = ["ChainError", "attn_bwd", "attn_bwd_workspace_bytes", "attn_fwd", "attn_partial",
           "library_path", "linear_attn_fwd", "linear_attn_workspace_bytes", "load", "lse_merge",
           "mlp_fwd", "mlp_fwd_noalloc", "mlp_gated_fwd", "mlp_workspace_bytes", "tile_census",
           "zigzag_segments"]
