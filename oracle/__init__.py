"""CPU oracle (test infrastructure only; see delta_rule.py)."""

from .delta_rule import (delta_rule_decode_step, delta_rule_forward, gated_delta_rule_decode_step,
                         gated_delta_rule_forward)
from .features import feature_maps, l2_normalize, round_to_bf16, sigmoid, silu
from .kda import kda_delta_rule_decode_step, kda_delta_rule_forward
from .backward import delta_rule_backward

__all__ = ["delta_rule_forward", "delta_rule_decode_step", "gated_delta_rule_forward",
           "gated_delta_rule_decode_step", "feature_maps", "l2_normalize", "round_to_bf16",
           "sigmoid", "silu", "kda_delta_rule_forward", "kda_delta_rule_decode_step",
           "delta_rule_backward"]
