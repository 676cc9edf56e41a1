"""Seeded synthetic inputs for the fused MoE forward pass.

This module is shared by the tests, the benchmark and the smoke check. It
holds input construction only -- random draws, dtype casts, the router
logits handed to the method as its input, expert-slot tables and per-slot
weight copies -- and none of the method's own arithmetic (no softmax, top-k,
masking, permutation, MLP or combine).
"""
from .configs import CONFIGS, WorkloadConfig, get_config
from .generate import (
    MoEInputs,
    bf16_round,
    build_slot_table,
    identity_slot_table,
    make_inputs,
    slot_weights,
)

__all__ = [
    "CONFIGS",
    "WorkloadConfig",
    "get_config",
    "MoEInputs",
    "bf16_round",
    "build_slot_table",
    "identity_slot_table",
    "make_inputs",
    "slot_weights",
]
