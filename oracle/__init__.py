"""CPU oracle of the fused MoE forward pass.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg. The HIP library never imports it.
"""
from .moe_oracle import (  # noqa: F401
    a2a_dispatch_indices,
    a2a_forward,
    combine_rows,
    ep_mask_and_remap,
    ep_partition,
    forward,
    forward_per_pair,
    grouped_down,
    grouped_gate_up,
    permute_indices,
    permute_rows,
    route,
    route_grouped,
    silu,
    slot_map,
    softmax,
    swiglu_mlp,
    topk_ids,
)
from .fp8_oracle import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    fp8_expert_mlp,
    fp8_forward,
    fp8_grouped_down,
    fp8_grouped_gate_up,
    fp8_linear,
    quantize_fp8,
)
