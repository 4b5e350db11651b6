"""MI355X-native single-GPU fine-grained MoE FFN layer forward.

Five steps, five C-ABI entry points in libmoe.so (declared in include/moe.h),
each wrapped here with the same name: moe_route, moe_dispatch,
moe_expert_ffn, moe_combine, moe_load_stats (moe_dispatch_capped is the
dispatch with expert capacities enforced; moe_expert_ffn_gather the FFN
reading token rows through the permutation, with no copy of them); and moe_bias_update, the
dynamic routing-bias step that feeds the next layer call. Every step runs in
the HIP kernels; this package only marshals tensors, sizes and the current stream.
"""
from .binding import (MoEError, MoELayerGraph, lib, moe_bias_update, moe_capacity, moe_combine,
                      moe_dispatch, moe_dispatch_noalloc, moe_expert_ffn, moe_expert_ffn_gather,
                      moe_layer_forward, moe_load_stats, moe_route, moe_status_string,
                      moe_dispatch_workspace_bytes, moe_expert_ffn_workspace_bytes,
                      moe_route_workspace_bytes)

__all__ = ["MoEError", "MoELayerGraph", "lib", "moe_route", "moe_dispatch",
           "moe_dispatch_noalloc", "moe_expert_ffn",
           "moe_expert_ffn_gather", "moe_combine",
           "moe_load_stats", "moe_bias_update", "moe_capacity", "moe_layer_forward", "moe_status_string",
           "moe_dispatch_workspace_bytes", "moe_expert_ffn_workspace_bytes",
           "moe_route_workspace_bytes"]
