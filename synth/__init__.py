"""Seeded synthetic-input generator shared by the tests, the benchmark and the oracle.

It makes inputs only and contains none of the method's arithmetic."""
from . import synth  # noqa: F401
