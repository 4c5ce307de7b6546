"""Seeded synthetic inputs for the packed-QKV split / per-head RMSNorm / RoPE path.

This module only draws random numbers and shapes them. It holds none of the
method's arithmetic (no split, no norm, no rotation), so both the CPU oracle
side and the HIP side of every test and of the benchmark can take their inputs
from here without sharing any of the computation.
"""
from .generators import (  # noqa: F401
    Workload,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    tiny_interleaved,
    decode_interleaved,
    prefill_interleaved,
    train_sectioned,
    latent_paged,
    gqa_paged,
    custom_gqa,
    token_positions,
    MlaDrafterInputs,
    mla_drafter_layer,
    SEEDS,
)
