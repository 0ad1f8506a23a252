"""fp64 CPU oracle for the single-GPU MoE-layer forward.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library
and its Python binding) never calls it and shares no code with it.
"""
from .moe_oracle import (  # noqa: F401
    router_logits,
    select_topk,
    route,
    selection_weights,
    e4m3_values,
    e4m3_encode,
    quantize_fp8,
    dequantize_fp8,
    MX_BLOCK,
    mx_scale_exponents,
    quantize_mx,
    dequantize_mx,
    expert_ffn_mx,
    capacity_slots,
    capacity_feasible,
    select_capacity,
    route_capacity,
    capacity_gaps,
    dispatch,
    silu,
    expert_ffn,
    grouped_ffn,
    shared_ffn,
    combine,
    forward,
    forward_tokens,
    dense_bruteforce,
    RouteResult,
    DispatchResult,
    ForwardResult,
)
