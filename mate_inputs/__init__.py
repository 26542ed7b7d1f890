"""Seeded synthetic inputs for the MATE token mixer, shared by the GPU tests,
the benchmark and the oracle tests.

This package holds shapes and random-number recipes only; it contains none of
the mixer's arithmetic (no scan, no decay, no attention).  Both the fp64 CPU
oracle and the HIP path consume exactly the arrays produced here.
"""
from .configs import MateShape, CONFIGS, config_shape, CONFIG_NOTES
from .generate import (
    MateInputs,
    make_inputs,
    make_block_inputs,
    make_block_weights,
    BLOCK_TENSOR_IDS,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    TENSOR_IDS,
)

__all__ = [
    "MateShape",
    "CONFIGS",
    "CONFIG_NOTES",
    "config_shape",
    "MateInputs",
    "make_inputs",
    "make_block_inputs",
    "make_block_weights",
    "BLOCK_TENSOR_IDS",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "TENSOR_IDS",
]
