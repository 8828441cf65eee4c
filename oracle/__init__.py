"""CPU oracle for the FP8-activation x block-scaled FP4 expert GEMM.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline leg are
the only callers.  Nothing in the product package imports this, and this imports nothing from it.
"""
from .oracle import *  # noqa: F401,F403
