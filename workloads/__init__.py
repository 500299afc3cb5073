"""Seeded synthetic inputs for the routed expert layer.

This package holds only input generation: shapes, seeds and random tensors.
It contains none of the layer's arithmetic (no routing, no expert FFN, no
cache policy), so both the HIP path and the CPU oracle can take their inputs
from here without sharing any computation.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from . import gen  # noqa: F401
