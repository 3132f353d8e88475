"""Seeded synthetic workloads for the SVDQuant linear layer and the INT8 KV-cache quantizer.

This package only draws random numbers and formats them as bf16 bit patterns. It holds none
of the quantization method's arithmetic, so both the CPU oracle and the GPU path may use it.
"""
from .workloads import (  # noqa: F401
    KV_CONFIG,
    LINEAR_CONFIGS,
    KVConfig,
    LinearConfig,
    bf16_bits_to_f32,
    f64_to_bf16_bits,
    make_bias,
    make_kv,
    make_linear,
    make_rng,
)
