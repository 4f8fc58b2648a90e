"""MI355X (gfx950) routed mixture-of-experts layer for speculative-decoding verify blocks
and prefill chunks.  The C ABI is ``include/moe.h``; this package is its Python binding.

Importing it requires the built HIP library (``libmoe_mi355x.so``); there is no CPU path.
"""
from ._lib import (  # noqa: F401
    Bank, Layer, MoeError, moe_align, moe_align_capacity, moe_align_workspace_size, moe_describe_plan,
    moe_experts_forward, moe_experts_workspace_size, moe_last_error, moe_layer_forward, moe_layer_forward_noalloc, moe_layer_workspace_size,
    moe_route_topk, moe_measure_stream_read, moe_set_stage_events, moe_workspace_status, stage_event_handles, moe_set_option, MOE_OPT_DECODE_FUSED, LIB_PATH, EXPORTS,
    MOE_W_BF16, MOE_W_FP8_E4M3, MOE_W_FP8_E4M3_A8, MOE_W_MXFP4,
)
