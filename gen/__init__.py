"""Seeded synthetic workloads (data only; no part of the method's arithmetic)."""
from . import synth, workloads  # noqa: F401
from .workloads import ALL, ALIASES, Workload, get, scaled  # noqa: F401
