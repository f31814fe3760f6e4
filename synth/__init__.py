"""Seeded synthetic inputs for the 4-bit MoE prefill layer.

This package is shared by the tests, the benchmark and the CPU oracle. It
only draws random tensors and prepares quantized expert weights the way an
offline model converter would (the workload recipe); it holds none of the
prefill computation itself (routing, permutation, dequantization, the expert
FFN or the combine).
"""
from .configs import CONFIGS, MoEConfig, get_config
from .gen import (
    LayerInputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_layer,
    make_stack_layer,
    make_tokens,
    pack_nibbles,
    quantize_asym,
    quantize_sym,
)

__all__ = [
    "CONFIGS",
    "MoEConfig",
    "get_config",
    "LayerInputs",
    "bf16_bits_to_f32",
    "f32_to_bf16_bits",
    "make_layer",
    "make_stack_layer",
    "make_tokens",
    "pack_nibbles",
    "quantize_asym",
    "quantize_sym",
]
