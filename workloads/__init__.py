"""Seeded synthetic inputs for the MXFP4 MoE expert layer.

This package only draws random numbers and lays them out.  It holds none of
the layer's arithmetic (no MX encoding, no routing, no FFN), so both the HIP
path and the CPU oracle can take their inputs from it without sharing any
method code.
"""
from .synth import (CONFIGS, Config, get_config, make_x_bf16, make_logits,
                    make_router_weight_bf16, make_weight_fp32, iter_weights_fp32,
                    bf16_bits_to_f32, make_shared_weight_fp32)

__all__ = ["CONFIGS", "Config", "get_config", "make_x_bf16", "make_logits",
           "make_router_weight_bf16", "make_weight_fp32", "iter_weights_fp32",
           "bf16_bits_to_f32", "make_shared_weight_fp32"]
