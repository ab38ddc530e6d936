"""Seeded synthetic workloads shared by the oracle, the tests and the benchmark."""
from .configs import WORKLOADS, Workload, decode, get  # noqa: F401
