"""Seeded synthetic decode workloads shared by the tests, the benchmark and the oracle checks.

This package only draws inputs (queries, KV caches, page tables, lengths, index lists). It holds
none of the attention or selection arithmetic: the CPU oracle and the HIP library each implement
that on their own and receive the tensors produced here.
"""

from .synth import (  # noqa: F401
    NAMED,
    Workload,
    make_named,
    make_workload,
    random_index_sets,
)
