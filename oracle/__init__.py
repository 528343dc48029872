"""CPU oracle for the bitplane-prefix expert path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product library.
"""
from .pm_oracle import *  # noqa: F401,F403
