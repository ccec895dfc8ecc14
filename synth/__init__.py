"""Seeded synthetic inputs for the DLRM hot path.

This package is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests.  It holds random-number generators, samplers and the workload
recipes only: no step of the model is computed here.
"""
from . import rng, workloads  # noqa: F401
