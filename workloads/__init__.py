"""Seeded synthetic serving mixes and the byte/FLOP accounting used to report them.

Holds none of the attention arithmetic: see synth.py for what it does build.
"""
from .synth import (  # noqa: F401
    BLOCK_SIZE, CONFIGS, SUPPLEMENTARY, SeqSpec, Workload, bf16_bits_to_f32, build, f32_to_bf16_bits, fp8_pool, make,
    pool_size_for,
)
from . import accounting  # noqa: F401
