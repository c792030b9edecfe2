"""Seeded synthetic inputs (tokens, Q/K/V, request traces) shared by the HIP
path's harness and the oracle. Holds no attention or cache arithmetic."""
from . import gen, configs  # noqa: F401
