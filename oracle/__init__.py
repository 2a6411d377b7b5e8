"""CPU oracle for the MXFP4 mixture-of-experts layer — TEST INFRASTRUCTURE.

Plain, slow, float64 NumPy code that states what the layer computes, used
only by the tests, by the smoke check and by the benchmark's CPU-baseline
leg.  The product path (the HIP library and its Python binding) never
imports, calls or links anything here.
"""
from .mxfp4_oracle import *  # noqa: F401,F403
