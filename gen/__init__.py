"""Seeded synthetic inputs, shared by the oracle checks, the GPU parity tests and
the benchmark.

This package only draws random numbers and lays them out in the shapes the
workloads use; it computes no part of the compression method itself.
"""
from .inputs import *  # noqa: F401,F403
