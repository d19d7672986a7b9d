"""Fused FlashAttention forward + Ulysses head-to-sequence re-layout on MI355X.

The compute path is libfa_relayout.so (hand-written gfx950 HIP kernels behind
the C ABI in include/fa_relayout.h); this package only builds it and binds it.
"""
from .binding import (FaError, LIB_PATH, attention_plain, attention_relayout,
                      attn_abi_version, attn_fwd_plain, attn_fwd_plain_async,
                      attn_fwd_plain_ws_async, attn_fwd_relayout, attn_fwd_relayout_async,
                      attn_fwd_relayout_ws_async, attn_fwd_slab_to_slab,
                      attn_fwd_slab_to_slab_async, attn_fwd_slab_to_slab_ws_async,
                      attn_fwd_workspace_bytes,
                      attn_status_string, load_library, relayout_to_slabs,
                      relayout_to_slabs_async)

__all__ = ["FaError", "LIB_PATH", "attention_plain", "attention_relayout",
           "attn_abi_version", "attn_fwd_plain", "attn_fwd_plain_async",
           "attn_fwd_plain_ws_async", "attn_fwd_relayout", "attn_fwd_relayout_async",
           "attn_fwd_relayout_ws_async", "attn_fwd_slab_to_slab",
           "attn_fwd_slab_to_slab_async", "attn_fwd_slab_to_slab_ws_async",
           "attn_fwd_workspace_bytes", "attn_status_string",
           "load_library", "relayout_to_slabs", "relayout_to_slabs_async"]
