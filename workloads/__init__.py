"""Seeded synthetic decode-attention workloads.

This package is the only code shared by the CPU oracle and the HIP path.  It
draws random numbers and lays them out; it holds none of the method's
arithmetic (no budgets, clusters, tiers, pages, quantisation or attention).
"""
from .gen import (  # noqa: F401
    Workload,
    make_workload,
    WORKLOAD_NAMES,
    bf16_round,
    bf16_bits_to_f32,
)
