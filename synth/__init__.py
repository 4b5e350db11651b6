"""Seeded synthetic workloads for the MoE FFN layer (inputs only, no layer arithmetic)."""
from .workloads import (CONFIGS, DECODE_TOKENS, MoEConfig, bf16_bits_to_f32, f32_to_bf16_bits,
                        make_layer, redraw_rows, get_config)

__all__ = ["CONFIGS", "DECODE_TOKENS", "MoEConfig", "bf16_bits_to_f32", "f32_to_bf16_bits",
           "make_layer", "redraw_rows", "get_config"]
