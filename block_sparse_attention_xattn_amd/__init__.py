"""MI355X (gfx950) XAttention block-sparse chunked prefill.

The compute path lives in libxattn.so (hand-written HIP kernels behind a C
ABI, declared in include/xattn.h).  ``binding`` marshals torch tensors into
those calls; ``prefill`` strings the calls into one layer's chunked prefill;
``synthetic`` draws seeded long-context inputs.
"""
from .binding import (XattnError, attn_merge, bsa_prefill, bsa_prefill_workspace_size,  # noqa: F401
                      xattn_estimate, xattn_estimate_workspace_size, xattn_mask_to_cache_blocks)

__all__ = ["XattnError", "attn_merge", "bsa_prefill", "bsa_prefill_workspace_size", "xattn_estimate",
           "xattn_estimate_workspace_size", "xattn_mask_to_cache_blocks"]
