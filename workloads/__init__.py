"""Seeded synthetic inputs for the Lookahead Sparse Attention (LSA) decode path.

This package only draws random numbers and lays them out.  It holds none of
the method's arithmetic (no query projection, no block scoring, no
threshold, no union, no attention): where an input has to be conditioned on
what the method computes (planted blocks that must score above the
threshold, keys redrawn away from the decision boundary) the caller passes
the needed functions in.  Both the oracle side (tests) and the GPU side
(tests, benchmark) build their inputs from here.
"""

from .configs import CONFIGS, LSAConfig, get_config
from .denoise import DenoiseWorkload, build_denoise_workload
from .gen import (
    Workload,
    bf16_bits_from_f32,
    build_workload,
    rng_for,
)

__all__ = [
    "CONFIGS",
    "DenoiseWorkload",
    "build_denoise_workload",
    "LSAConfig",
    "get_config",
    "Workload",
    "bf16_bits_from_f32",
    "build_workload",
    "rng_for",
]
