"""Seeded synthetic workload generators (random numbers only)."""
from . import gen  # noqa: F401
