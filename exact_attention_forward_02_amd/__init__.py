"""Fused exact-attention forward for AMD Instinct MI355X (gfx950).

``attn_fwd(q, k, v, causal=False, scale=None) -> (o, lse)`` runs the
hand-written HIP kernel through the C ABI in include/attn_fwd.h;
``attn_fwd_ex`` takes strided views (e.g. [B, S, H, d] layouts) in bf16 or
fp16; ``attn_bwd`` computes the gradients by recomputation from lse, and
``attn_bwd_noalloc`` does the same without any device allocation.  The
split-key path (``attn_fwd_split``, ``attn_merge``, ``attn_fwd_splitkv``)
computes the same result from per-split states merged afterwards; with at
most 16 query rows per K/V head the per-split states come from a key-streaming
decode kernel (``attn_fwd_decode``).
``attn_fwd_varlen`` runs a packed batch of sequences of different lengths on
the schedule ``varlen_plan`` computes on the host.
"""
from ._binding import (attn_bwd, attn_bwd_noalloc, attn_fwd, attn_fwd_dbg,  # noqa: F401
                       attn_fwd_decode, attn_fwd_ex, attn_fwd_split, attn_fwd_splitkv,
                       attn_fwd_varlen, attn_merge, library, split_keys, status_string,
                       varlen_plan)

__all__ = ["attn_fwd", "attn_fwd_dbg", "attn_fwd_ex", "attn_bwd", "attn_bwd_noalloc",
           "attn_fwd_split",
           "attn_fwd_decode",
           "attn_merge", "attn_fwd_splitkv", "attn_fwd_varlen", "varlen_plan", "split_keys",
           "library", "status_string"]
