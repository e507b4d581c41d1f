"""MI355X (gfx950) DeepSeekMoE layer forward pass.

The compute lives in ``libmoe_layer.so`` (hand-written HIP kernels behind the
C ABI of ``include/moe_layer.h``); this package is its Python binding.
"""
from ._lib import (MOE_BF16, MOE_FP8, MOE_ERR_ALIAS, MOE_ERR_HIP, MOE_ERR_INVALID_ARG,
                   MOE_ERR_SCRATCH, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_F32, MOE_OK,
                   NOALLOC_SCRATCH_BYTES,
                   HipEvents, MoeError, MoeLayerDesc, header_functions,
                   backward_stage_names, backward_workspace_size, load_library, make_desc, moe_bias_update,
                   moe_layer_backward, moe_layer_forward, moe_layer_forward_noalloc,
                   quantize_fp8_blocks, side_stream_count, strerror,
                   trace_stage_names, validate, workspace_layout,
                   workspace_size)

__all__ = [
    "MOE_BF16", "MOE_FP8", "MOE_ERR_ALIAS", "MOE_ERR_HIP", "MOE_ERR_INVALID_ARG",
    "MOE_ERR_SCRATCH", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MOE_F32", "MOE_OK",
    "NOALLOC_SCRATCH_BYTES",
    "HipEvents", "MoeError", "MoeLayerDesc", "header_functions",
    "backward_stage_names", "backward_workspace_size", "load_library", "make_desc", "moe_bias_update",
    "moe_layer_backward", "moe_layer_forward", "moe_layer_forward_noalloc",
    "quantize_fp8_blocks", "side_stream_count", "strerror",
    "trace_stage_names", "validate", "workspace_layout", "workspace_size",
]
