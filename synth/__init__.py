"""Seeded synthetic inputs shared by the CPU oracle's tests and the HIP path's tests and bench.

This package only draws random numbers and lays them out (bf16 rounding, page scatter).  It holds
none of the method's arithmetic: no prediction, scoring, selection or attention happens here.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
