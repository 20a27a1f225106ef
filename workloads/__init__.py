"""Seeded synthetic workloads shared by the tests, the bench and the oracle checks.

This package holds shapes and random inputs only; none of the attention
arithmetic lives here.
"""
from .gen import Workload, WORKLOADS, make_workload, generate, Inputs  # noqa: F401
