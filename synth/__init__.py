"""Seeded synthetic video-token inputs (Q, K, V on a T x Hh x W latent grid).

This module only draws random numbers and lays them out. It holds none of the
block-sparse attention arithmetic, so both the CPU oracle side (tests, the
bench's CPU baseline) and the GPU side (tests, bench) can take their inputs
from it without sharing any of the method's code.
"""
from .video import (
    Config,
    CONFIGS,
    TEST_CONFIGS,
    get_config,
    make_inputs,
    bf16_bits_to_f64,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
)

__all__ = [
    "Config",
    "CONFIGS",
    "TEST_CONFIGS",
    "get_config",
    "make_inputs",
    "bf16_bits_to_f64",
    "bf16_bits_to_f32",
    "f32_to_bf16_bits",
]
