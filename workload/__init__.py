"""Seeded synthetic workloads for the BlockFFN layer and the FFF tree layer.

This package is the one source of inputs shared by the CPU oracle's tests, the
GPU parity tests, ``smoke()`` and ``bench.py``.  It draws weights and tokens
and nothing else: it holds none of the layer's arithmetic (no router, no
experts, no union), so neither side of a parity check can borrow it from the
other through here.
"""
from .configs import CONFIGS, WorkloadConfig, get_config
from .gen import Layer, Tokens, make_layer, make_tokens, make_workload, bf16_round_bits, bf16_bits_to_f32
from .fff import (FFF_CONFIGS, FffConfig, FffLayer, get_fff_config, make_fff_layer, make_fff_tokens,
                  make_fff_workload)

__all__ = [
    "CONFIGS", "WorkloadConfig", "get_config", "Layer", "Tokens", "make_layer",
    "make_tokens", "make_workload", "bf16_round_bits", "bf16_bits_to_f32",
    "FFF_CONFIGS", "FffConfig", "FffLayer", "get_fff_config", "make_fff_layer", "make_fff_tokens",
    "make_fff_workload",
]
