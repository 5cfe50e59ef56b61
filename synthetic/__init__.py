"""Seeded synthetic workload generator (no layer arithmetic)."""
from .gen import CONFIGS, MoEConfig, MoEInputs, make_inputs, f32_to_bf16_bits

__all__ = ["CONFIGS", "MoEConfig", "MoEInputs", "make_inputs", "f32_to_bf16_bits"]
