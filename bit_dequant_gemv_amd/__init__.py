"""MI355X-native sparse-MoE expert decode over MXFP4 / packed-int4 weights,
with the decode attention of a gpt-oss layer beside it.

The compute lives in ``libbdg.so`` (HIP kernels for gfx950, C ABI in
``include/bdg.h``); this package is its thin Python binding.
"""

from .api import (KERNEL_KINDS, KernelTimes, MoEPlan, QWeight, attn_decode, attn_decode_noalloc,
                  attn_decode_workspace_bytes, attn_rope_table, attn_workspace, int4g_dequant, moe_expert_decode,
                  moe_expert_decode_profiled, moe_expert_decode_timeline, moe_experts_routed,
                  moe_prefill_mx, moe_router_topk, mx_gemm, mx_gemm_workspace_bytes, mxfp4_dequant,
                  mxfp8_quantize, prefill_workspace_bytes, prefill_workspace_views, qgemv, stream_copy,
                  stream_read, version)

__all__ = [
    "KERNEL_KINDS", "KernelTimes", "MoEPlan", "QWeight", "attn_decode", "attn_decode_noalloc",
    "attn_decode_workspace_bytes", "attn_rope_table", "attn_workspace", "int4g_dequant", "moe_expert_decode",
    "moe_expert_decode_profiled", "moe_expert_decode_timeline", "moe_experts_routed",
    "moe_prefill_mx", "moe_router_topk", "mx_gemm", "mx_gemm_workspace_bytes", "mxfp4_dequant", "mxfp8_quantize",
    "prefill_workspace_bytes", "prefill_workspace_views", "qgemv", "stream_copy", "stream_read",
    "version",
]
