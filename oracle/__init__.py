"""CPU float64 oracle of the predictor-gated sparse FFN.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .pi_oracle import *  # noqa: F401,F403
