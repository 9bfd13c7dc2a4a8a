"""Seeded synthetic workloads for sparse-linear attention.

This package is shared by the tests, the benchmark and the smoke check.  It
holds only input synthesis (shapes, counts, random draws); none of the
method's arithmetic lives here, so the CPU oracle and the HIP path can both
consume its tensors without sharing any computation.
"""
from .synth import (  # noqa: F401
    Workload,
    CONFIGS,
    band_count,
    make_workload,
    make_custom,
    num_blocks,
)
