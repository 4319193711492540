"""Synthetic workload presets and seeded input generators (shared by the GPU harness and
the CPU oracle's tests; no part of the method's arithmetic lives here)."""
from .configs import WORKLOADS, LatencyModel, ModelShape, Workload, scaled  # noqa: F401
