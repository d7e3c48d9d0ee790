"""Seeded synthetic workloads for the dropless MoE layer forward pass.

This package only draws random numbers and fixes shapes.  It holds none of the
layer's arithmetic (no routing, no counting, no matrix products), so that both
the HIP path and the CPU oracle can take their inputs from it without sharing
any of the method's code.
"""
from .configs import CONFIGS, MoEConfig, get_config  # noqa: F401
from .gen import make_inputs, make_fp8_weights, MoEInputs, Fp8Weights  # noqa: F401
