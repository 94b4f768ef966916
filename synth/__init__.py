"""Seeded synthetic input generators shared by the oracle tests, the GPU tests
and the benchmark. Holds no route arithmetic."""
from . import generators  # noqa: F401
