"""Seeded synthetic MoE routing workloads shared by the tests and the benchmark.

This package holds input generation only: no layout, dispatch or combine
arithmetic.  The oracle and the HIP library both consume the arrays it makes.
"""

from .workloads import CONFIGS, Workload, algorithmic_bytes, make_workload, zipf_probs

__all__ = ["CONFIGS", "Workload", "algorithmic_bytes", "make_workload", "zipf_probs"]
