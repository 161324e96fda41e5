"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This package draws random numbers and rounds them to bf16; it holds none of
the arithmetic of the method itself.
"""
from .grpo_inputs import (  # noqa: F401
    CONFIGS,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    make_config,
    make_case,
)
