"""4-bit block-quantized MoE prefill on AMD MI355X (gfx950).

The computation lives in the HIP library libqmoe.so (C ABI in include/moe.h);
this package is its Python binding. Importing the package does not load the
library; the first call does, and fails loudly if it has not been built.
"""
from ._native import (MOE_OK, MOE_ERR_HIP, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED,
                      MOE_ERR_WORKSPACE_TOO_SMALL, MOE_WS_EXPERT_FFN, MOE_WS_EXPERT_FFN_I8,
                      MOE_WS_LAYER, MOE_WS_LAYER_I8, MOE_WS_PERMUTE, MOE_WS_ROUTE,
                      MOE_STATIC_WS_BYTES, MOE_W_ROWS, MOE_W_TILED, MoeError, lib)
from .ops import (Experts, MixedExperts, MoELayer, MoEStack, StreamedExperts, make_shape,
                  moe_combine, moe_layer_forward_streamed, moe_stream_stage_bytes,
                  moe_expert_ffn, moe_expert_ffn_i8, moe_expert_ffn_mixed, moe_layer_forward,
                  moe_layer_forward_static,
                  moe_layer_forward_i8, moe_layer_forward_mixed, moe_permute,
                  moe_pack_tier, moe_pack_w4, moe_quantize_rows_i8, moe_rmsnorm, moe_route, moe_workspace_size,
                  pack_layer, pack_mixed, profile_enable, profile_read, profile_reset, shape_of, workspace)

__all__ = [
    "MOE_OK", "MOE_ERR_HIP", "MOE_ERR_INVALID_ARGUMENT", "MOE_ERR_UNSUPPORTED",
    "MOE_ERR_WORKSPACE_TOO_SMALL", "MOE_WS_EXPERT_FFN", "MOE_WS_EXPERT_FFN_I8", "MOE_WS_LAYER",
    "MOE_WS_LAYER_I8", "MOE_WS_PERMUTE", "MOE_WS_ROUTE", "MoeError", "lib", "Experts", "MixedExperts", "MoELayer", "StreamedExperts",
    "moe_layer_forward_streamed", "moe_stream_stage_bytes",
    "MOE_W_ROWS", "MOE_W_TILED", "moe_pack_w4", "moe_pack_tier", "pack_layer", "pack_mixed",
    "MoEStack", "make_shape", "moe_combine", "moe_expert_ffn", "moe_expert_ffn_i8", "moe_expert_ffn_mixed",
    "moe_layer_forward", "moe_layer_forward_static", "MOE_STATIC_WS_BYTES", "moe_layer_forward_mixed", "moe_layer_forward_i8", "moe_permute", "moe_quantize_rows_i8",
    "moe_rmsnorm", "moe_route", "moe_workspace_size", "profile_enable", "profile_read",
    "profile_reset", "shape_of", "workspace",
]
