"""Seeded synthetic inputs for the block-sparse decode path.

This package only draws random numbers and lays them out in the tensor shapes
the workloads use.  It holds none of the method's arithmetic (no pooling, no
scoring, no selection, no attention), so the CPU oracle and the HIP path can
both be fed from it without sharing any computation.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from . import inputs  # noqa: F401
