"""CPU oracle of the MoE expert-layer forward — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The GPU path never calls it and shares no code with it.
"""
from .moe import (  # noqa: F401
    expert_range,
    route_topk,
    dispatch,
    silu,
    swiglu_hidden,
    expert_ffn,
    grouped_experts,
    combine,
    moe_layer,
    brute_force_dense,
    token_outputs,
)
