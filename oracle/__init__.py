"""CPU fp64 oracle for packed joint attention with Q/K RMSNorm and 3-axis RoPE.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, calls or links anything under ``oracle/``; only
the tests, the smoke check and the CPU-baseline leg of the benchmark do.

See :mod:`oracle.attention` for the definitions and their citations.
"""
from .attention import *  # noqa: F401,F403
