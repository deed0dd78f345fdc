"""WIDE masked dynamic-width execution on MI355X (gfx950).

A thin Python binding over ``libwide.so``, the C ABI declared in
``include/wide.h``.  The functions here only marshal arguments (torch tensors
-> device pointers, shapes, the current HIP stream) and raise on a non-zero
status; every step of the computation runs in the HIP kernels of the library.
There is no fallback: without the built library, or without a GPU, the calls
raise.
"""
from .binding import (LIB_PATH, WideError, attn_decode_masked_cache, attn_decode_masked_paged,
                      attn_proj_masked,
                      attn_proj_masked_workspace,
                      ffn_masked, ffn_masked_f32, ffn_masked_f32_workspace, ffn_masked_noalloc,
                      ffn_masked_workspace, layer_decode_masked_cache,
                      layer_decode_masked_paged, layer_masked, layer_masked_routed,
                      layer_masked_workspace, mask_reorder_packed,
                      lib, mask_reorder, pack_kmajor, pack_router, router_topk, trace_collect,
                      trace_enable, trace_reset, WIDE_DECODE, WIDE_PREFILL)

__all__ = [
    "LIB_PATH", "WideError", "lib", "mask_reorder", "pack_kmajor", "pack_router", "router_topk",
    "ffn_masked", "ffn_masked_f32", "ffn_masked_f32_workspace", "ffn_masked_noalloc",
    "ffn_masked_workspace", "attn_proj_masked", "attn_proj_masked_workspace",
    "attn_decode_masked_cache", "attn_decode_masked_paged", "layer_masked", "layer_masked_routed",
    "layer_decode_masked_cache", "layer_decode_masked_paged", "mask_reorder_packed",
    "layer_masked_workspace", "trace_enable", "trace_reset", "trace_collect", "WIDE_PREFILL",
    "WIDE_DECODE",
]
