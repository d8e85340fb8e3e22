"""Seeded synthetic inputs shared by the CPU oracle's tests and the HIP path.

This package only synthesises inputs (sequence lengths, block placement, N(0,1)
values rounded to a storage dtype). It holds none of the attention arithmetic.
"""
from .gen import *  # noqa: F401,F403
