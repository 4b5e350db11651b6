"""CPU oracle of the MoE FFN layer forward: test infrastructure only."""
from .moe_oracle import (widen, logits, route, dispatch, gelu_erf, expert_ffn, expert_outputs,
                         shared_outputs, combine, layer, layer_rows, load_stats, gini_page_formula,
                         load_fraction, prob_mean, bias_update, capacity, dispatch_capped,
                         kept_mask)

__all__ = ["widen", "logits", "route", "dispatch", "gelu_erf", "expert_ffn", "expert_outputs",
           "shared_outputs", "combine", "layer", "layer_rows", "load_stats", "gini_page_formula",
           "load_fraction", "prob_mean", "bias_update", "capacity", "dispatch_capped",
           "kept_mask"]
