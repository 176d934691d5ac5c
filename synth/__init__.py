"""Seeded synthetic inputs for the MoE routing/dispatch path.

This package only draws random numbers and lays them out in the shapes of the
five model-shaped workloads. It holds none of the routing arithmetic: no
gate, no top-K, no sort, no reduction. Both the CPU oracle's tests and the GPU
benchmark feed from it, so they see byte-identical inputs for a given seed.

bf16 tensors are carried as ``numpy.uint16`` bit patterns (the upper half of
an IEEE binary32). The float -> bf16 encoding here uses PyTorch's CPU
conversion (round to nearest even); it is data encoding, not method
arithmetic.
"""

from .configs import CONFIGS, RouteConfig, PredictorConfig, FoEConfig, get_config
from .gen import (
    zipf_ids,
    to_bf16_bits,
    from_bf16_bits,
    make_route_inputs,
    make_foe_inputs,
    make_predictor_layer,
    make_config_inputs,
    first_tokens,
    default_expert_cluster,
    foe_row_cluster,
)

__all__ = [
    "CONFIGS",
    "RouteConfig",
    "PredictorConfig",
    "FoEConfig",
    "get_config",
    "zipf_ids",
    "to_bf16_bits",
    "from_bf16_bits",
    "make_route_inputs",
    "make_foe_inputs",
    "make_predictor_layer",
    "make_config_inputs",
    "first_tokens",
    "default_expert_cluster",
    "foe_row_cluster",
]
