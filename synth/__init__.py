"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package holds no arithmetic of the MoE layer itself: only random draws,
the encodings of those draws into the stored formats (f32, bf16, MXFP4 bits)
and the packing of one expert's matrices into its slot byte layout.
"""
from .gen import *  # noqa: F401,F403
from .configs import *  # noqa: F401,F403
