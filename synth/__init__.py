"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package only draws random numbers. It holds none of the method's
arithmetic: no packing, no quantization, no routing, no dot products.
"""
from .gen import *  # noqa: F401,F403
