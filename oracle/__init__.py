"""CPU oracle of the Muon step.  Test infrastructure only: imported by tests/,
the smoke check and the benchmark's CPU-baseline leg, never by the library."""

from .muon_oracle import *  # noqa: F401,F403
from . import muon_oracle  # noqa: F401
