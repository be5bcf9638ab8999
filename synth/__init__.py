"""Seeded synthetic workloads (shapes, weights, tokens, bias) for the sparse FFN.

Shared by the oracle-side tests and the GPU side.  Holds none of the method's
arithmetic.
"""
from . import configs, gen  # noqa: F401
