"""Fused exact-attention forward for AMD Instinct MI355X (gfx950).

``attn_fwd(q, k, v, causal=False, scale=None) -> (o, lse)`` runs the
hand-written HIP kernel through the C ABI in include/attn_fwd.h.
"""
from ._binding import attn_fwd, attn_fwd_dbg, library, status_string  # noqa: F401

__all__ = ["attn_fwd", "attn_fwd_dbg", "library", "status_string"]
