"""Seeded synthetic inputs for the CSA/HCA attention path.

This package is shared by the tests, the benchmark and the oracle.  It only
draws random numbers and encodes them into the storage formats the path
consumes (bf16, fp8-e4m3fn, MXFP4); it performs none of the attention
method's arithmetic.
"""
from .configs import CONFIGS, LayerConfig, get_config  # noqa: F401
from . import gen, encode  # noqa: F401
