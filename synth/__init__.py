"""Seeded synthetic inputs for the Orthrus draft/verify step.

This package is the only code shared by the CPU oracle and the HIP path.  It
draws random numbers and lays them out in memory; it performs none of the
method's arithmetic (no attention, no argmax, no acceptance, no commit).
"""
from .inputs import *  # noqa: F401,F403
