"""CPU oracle of the MoE expert-layer forward and its gradient — TEST INFRASTRUCTURE ONLY.

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
from .moe_backward import (  # noqa: F401
    silu_grad,
    route_topk_backward,
    combine_backward,
    swiglu_backward,
    expert_ffn_backward,
    dispatch_backward,
    moe_layer_backward,
)
