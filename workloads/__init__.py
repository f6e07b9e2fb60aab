"""Seeded synthetic inputs for the MoE-layer forward.

This package holds no step of the MoE method: only shapes, seeds and the
recipes that draw x, W_gate and the expert weights.  Both the HIP path and
the CPU oracle are fed from it, with the same bits.
"""
from .configs import CONFIGS, MoEConfig, get_config  # noqa: F401
from .synth import (  # noqa: F401
    bf16_bits_to_f32,
    expert_stack,
    expert_weight,
    f32_to_bf16_bits,
    router_inputs,
    storage_bits,
)
