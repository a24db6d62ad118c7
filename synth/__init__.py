"""Seeded synthetic inputs shared by the GPU tests, the oracle tests and the
benchmark.  Holds none of the mixer's arithmetic: only random draws, the
rounding of those draws to the storage dtype, and the workload table."""
from .inputs import *  # noqa: F401,F403
