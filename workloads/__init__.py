"""Seeded synthetic workloads for the quantized-KV decode path.

This package holds only input generation (shapes, value distributions, seeds, page tables).
It contains none of the method's arithmetic, and it is the one piece shared by the oracle
tests, the GPU tests and the benchmark.
"""
from .configs import CONFIGS, Workload  # noqa: F401
from . import generate  # noqa: F401
