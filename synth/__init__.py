"""Seeded synthetic inputs shared by the oracle and the HIP path (no layer arithmetic)."""
from .cases import (SHAPES, LayerShape, LayerInputs, MARGIN, custom_shape, make_inputs,
                    expert_weights, all_expert_weights_host, f32_to_bf16_bits, bf16_bits_to_f32)

__all__ = ["SHAPES", "LayerShape", "LayerInputs", "MARGIN", "custom_shape", "make_inputs",
           "expert_weights", "all_expert_weights_host", "f32_to_bf16_bits", "bf16_bits_to_f32"]
