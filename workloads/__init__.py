"""Seeded synthetic inputs shaped like the decode-step workloads (shared by tests, smoke, bench)."""
from .synth import WORKLOADS, Workload, make  # noqa: F401
