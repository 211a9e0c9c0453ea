"""Seeded synthetic inputs for the compressed linear layer forward.

This package only draws random numbers and rounds them to the storage
types of the format (fp16, bf16, small integers).  It holds none of the
forward's arithmetic: no dequantisation, no reconstruction, no product.
Both the CPU oracle and the HIP path consume what it produces.
"""
from .layers import (
    LogicalLayer,
    CONFIGS,
    config_layers,
    make_layer,
    make_x,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
)

__all__ = [
    "LogicalLayer",
    "CONFIGS",
    "config_layers",
    "make_layer",
    "make_x",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
]
