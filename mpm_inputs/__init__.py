"""Seeded synthetic inputs shared by the oracle tests, the HIP library's
tests and the benchmark.  Holds no part of the transfer's arithmetic."""
from . import generators
from .workloads import WORKLOADS, Workload, build, scaled

__all__ = ["generators", "WORKLOADS", "Workload", "build", "scaled"]
