"""MI355X (gfx950) MXFP4 block-scaled MoE layer and dense projections.

The compute path is libmxfp4moe.so (hand-written HIP kernels behind the C ABI
in include/mxfp4_moe.h); this package is its thin ctypes binding.  Build the
library with ``__graft_entry__.build()`` or ``python -m
mxfp4_block_scaled_top_amd.build``.
"""

from ._lib import (ACT_BF16, ACT_FP8_E4M3, ACT_MXFP4, LIB_PATH, NUM_STAGES, STAGES,  # noqa: F401
                   Mxfp4Error, lib, mxfp4_abi_version, mxfp4_event_create,
                   mxfp4_event_destroy, mxfp4_event_elapsed_ms, mxfp4_linear,
                   mxfp4_linear_workspace_size,
                   mxfp4_moe_code_stream_size, mxfp4_moe_forward, mxfp4_moe_layer,
                   mxfp4_moe_layer_noalloc, mxfp4_moe_prepare_code_stream,
                   mxfp4_moe_workspace_layout_query,
                   mxfp4_moe_workspace_size, mxfp4_quant_fp8_e4m3, mxfp4_quantize_weights,
                   mxfp4_route_topk, mxfp4_stream_read, nvfp4_moe_forward,
                   nvfp4_moe_workspace_size)
