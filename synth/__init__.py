"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This package draws random numbers and shapes them into test workloads. It
holds none of the block-sparse attention arithmetic: no layout, scoring,
selection or attention code lives here, and it imports nothing from
``oracle`` or ``video_diffusion_block_amd``.
"""
from .fields import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_to_f32,
    bf16_bits_to_f64,
    f32_to_bf16_bits,
    gaussian_noise,
    make_inputs,
    smooth_field,
)
