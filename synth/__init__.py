"""Seeded synthetic inputs for the NVFP4 MoE path (shared by tests, bench and the oracle's callers).

This package draws random inputs only. It holds none of the method's arithmetic: no decoding of
E2M1 / E4M3, no GEMM, no routing plan. Both the HIP library's callers and the oracle's callers
take their inputs from here.
"""
from .inputs import *  # noqa: F401,F403
