"""Seeded synthetic inputs for the MoE layer forward.

Shared by the oracle side (tests, CPU baseline) and the GPU side (tests, bench):
it draws data and holds none of the layer's arithmetic.
"""
from .configs import CONFIGS, MoEConfig, config
from .generate import FP8_BLOCK, generate, rng, to_bf16_bits, to_e4m3_codes

__all__ = ["CONFIGS", "MoEConfig", "config", "generate", "rng", "FP8_BLOCK",
           "to_bf16_bits", "to_e4m3_codes"]
