"""Seeded synthetic workloads for the routed-expert MoE FFN layer.

This package only draws random inputs (weights, tokens, noise, reuse coins) in
the canonical host layout.  It holds none of the layer's arithmetic, so both the
GPU path and the fp64 oracle can consume its arrays without sharing code.
"""
from .workloads import (  # noqa: F401
    WORKLOADS, Workload, make_layer, make_tokens, make_noise, make_reuse_coins,
    f32_to_bf16_bits, bf16_bits_to_f32, layer_bytes, expert_bytes,
)
