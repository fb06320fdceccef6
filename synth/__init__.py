"""Seeded synthetic inputs (configurations, token streams, weights).

This module is shared by the float64 oracle and by the GPU path. It holds
none of the method's arithmetic: it only draws random numbers and plants
repeated segments, so neither side can inherit a mistake from the other.
"""
from .gen import CONFIGS, config, gen_tokens, gen_weights, weight_names, weight_shapes, n_weights

__all__ = ["CONFIGS", "config", "gen_tokens", "gen_weights", "weight_names",
           "weight_shapes", "n_weights"]
