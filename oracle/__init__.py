"""fp64 CPU oracle of the Periodic Row-wise Muon step.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library or its binding.
"""
from .muon_oracle import *  # noqa: F401,F403
from .muon_oracle import __all__  # noqa: F401
