"""Seeded synthetic inputs for the ReDrafter verification step.

This package only draws random numbers and lays them out.  It holds none of
the verification arithmetic (no packing, masking, attention, projection,
unpacking or acceptance); the CPU oracle and the HIP path both receive the
arrays it returns.
"""
from .gen import *  # noqa: F401,F403
