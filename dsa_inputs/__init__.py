"""Seeded synthetic inputs for the sparse-attention workloads.

Shared by the oracle tests and the GPU path's tests and bench; holds only
random draws and storage rounding, none of the method's arithmetic.
"""
from . import gen, configs  # noqa: F401
from .configs import WORKLOADS, Workload  # noqa: F401
