"""MI355X-native forward pass of one MoE feed-forward layer (route, permute,
grouped FFN, combine) as HIP kernels behind a C ABI (include/moe.h).

This package is the thin Python binding of ``libmoe.so``; torch provides
device memory and streams only.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    MOE_BF16,
    MOE_ERR_HIP,
    MOE_ERR_INVALID_ARG,
    MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE,
    MOE_F32,
    MOE_OK,
    MoEError,
    load_library,
    moe_combine,
    moe_ffn_workspace_bytes,
    moe_forward,
    moe_forward_fp8,
    moe_fp8_weight_bytes,
    moe_grouped_ffn,
    moe_grouped_ffn_fp8,
    moe_grouped_ffn_padded,
    moe_pad_dispatch,
    moe_permute,
    moe_permute_workspace_bytes,
    moe_quantize_fp8,
    moe_route,
    moe_route_capacity,
    moe_route_workspace_bytes,
    moe_select_capacity,
    moe_workspace_bytes,
    strerror,
    version,
)
