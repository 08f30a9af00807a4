"""MI355X (gfx950) XAttention block-sparse chunked prefill.

The compute path lives in libxattn.so (hand-written HIP kernels behind a C
ABI, declared in include/xattn.h).  ``binding`` marshals torch tensors into
those calls; ``prefill`` strings the calls into one layer's chunked prefill;
``synthetic`` draws seeded long-context inputs.
"""
from .binding import (PackedV, XattnError, attn_merge, bsa_pack_v, bsa_packed_v_bytes,  # noqa: F401
                      bsa_prefill, bsa_prefill_packed, bsa_prefill_packed_workspace_size, bsa_prefill_segments,
                      bsa_prefill_segments_workspace_size, bsa_prefill_workspace_size, xattn_estimate,
                      xattn_estimate_workspace_size, xattn_mask_to_cache_blocks, xattn_downsample_keys,
                      xattn_estimate_history_ds, xattn_estimate_history_ds_workspace_size, OffloadedKV,
                      xattn_offload_blocks, bsa_history_offloaded, xattn_estimate_offloaded,
                      xattn_varlen_mask_elems, xattn_estimate_varlen, xattn_estimate_varlen_workspace_size,
                      bsa_prefill_varlen, bsa_prefill_varlen_workspace_size, varlen_blocks, varlen_lse)

__all__ = ["PackedV", "XattnError", "attn_merge", "bsa_pack_v", "bsa_packed_v_bytes", "bsa_prefill",
           "bsa_prefill_packed", "bsa_prefill_packed_workspace_size", "bsa_prefill_segments",
           "bsa_prefill_segments_workspace_size", "bsa_prefill_workspace_size", "xattn_estimate",
           "xattn_estimate_workspace_size", "xattn_mask_to_cache_blocks", "xattn_downsample_keys",
           "xattn_estimate_history_ds", "xattn_estimate_history_ds_workspace_size", "OffloadedKV",
           "xattn_offload_blocks", "bsa_history_offloaded", "xattn_estimate_offloaded", "xattn_varlen_mask_elems",
           "xattn_estimate_varlen", "xattn_estimate_varlen_workspace_size", "bsa_prefill_varlen",
           "bsa_prefill_varlen_workspace_size", "varlen_blocks", "varlen_lse"]
