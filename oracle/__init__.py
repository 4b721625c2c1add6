"""CPU oracle of the AuT encoder forward pass -- test infrastructure only.

Used by tests/, the smoke check and the benchmark's CPU-baseline leg; the
HIP product path never imports or calls it.  Everything is float64 numpy.
"""
from .aut_oracle import *  # noqa: F401,F403
