"""Seeded synthetic inputs for the Mixtral MoE feed-forward layer.

This package is the only code shared by the CPU oracle and the GPU path.  It
draws inputs (activations, router and expert weights, router bias, and the
attention sublayer's activations and projections) from fixed
distributions and seeds and holds none of the layer's arithmetic.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    MoEConfig,
    attention_heads,
    attention_inputs,
    bf16_bits_from_f32,
    config_by_name,
    generate,
    generate_torch,
    zipf_router_bias,
)
