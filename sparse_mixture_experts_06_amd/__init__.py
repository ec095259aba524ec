"""Mixtral sparse-MoE feed-forward layer for AMD Instinct MI355X (gfx950).

The layer runs in libmoe.so (hand-written HIP kernels behind the C ABI in
include/moe.h); this package is its Python binding. The library is loaded on
first use (or by load()), and every call raises if it has not been built;
there is no fallback.
"""
from ._lib import (MOE_BF16, MOE_BF16_PACKED, MOE_EHIP, MOE_EINVAL, MOE_ENOTSUP, MOE_EWORKSPACE,
                   MOE_F32, MOE_INT8_PACKED, MOE_MAX_ASSIGNMENTS, MOE_MAX_EXPERTS,
                   MOE_NOALLOC_SCRATCH_BYTES, MOE_OK,
                   MoeError, MoeOptions, PackedWeights, QuantizedMatrix, QuantizedWeights,
                   header_functions, load, moe_block_forward, moe_check_routing, moe_combine,
                   moe_expert_ffn,
                   moe_forward, moe_forward_noalloc, moe_pack_weight, moe_permute, moe_quantize_weight, moe_route,
                   moe_workspace_bytes, strerror, workspace)

__all__ = ["MOE_BF16", "MOE_BF16_PACKED", "MOE_EHIP", "MOE_EINVAL", "MOE_ENOTSUP",
           "MOE_EWORKSPACE", "MOE_F32", "MOE_INT8_PACKED", "MOE_MAX_ASSIGNMENTS",
           "MOE_MAX_EXPERTS", "MOE_NOALLOC_SCRATCH_BYTES", "MOE_OK", "MoeError", "MoeOptions", "PackedWeights",
           "QuantizedMatrix", "QuantizedWeights", "header_functions", "load",
           "moe_block_forward", "moe_check_routing", "moe_combine", "moe_expert_ffn", "moe_forward", "moe_forward_noalloc",
           "moe_pack_weight", "moe_permute", "moe_quantize_weight", "moe_route",
           "moe_workspace_bytes", "strerror", "workspace"]
