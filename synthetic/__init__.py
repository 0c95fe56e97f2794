"""Seeded synthetic inputs for permuted block-sparse prefill attention.

This package holds no arithmetic of the attention method. It only draws
random tensors with planted stripe structure and rounds them to bfloat16
bit patterns, so that the CPU oracle and the GPU path consume identical
inputs.
"""
from .stripes import (StripeSpec, make_stripe_inputs, round_to_bf16_bits,
                      bf16_bits_to_float32)
from .configs import CONFIGS, get_config, WorkloadConfig

__all__ = ["StripeSpec", "make_stripe_inputs", "round_to_bf16_bits",
           "bf16_bits_to_float32", "CONFIGS", "get_config", "WorkloadConfig"]
