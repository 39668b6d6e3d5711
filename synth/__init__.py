"""Seeded synthetic inputs for paged decode attention.

This module only draws and lays out inputs (query rows, a paged KV pool, block
tables, lengths, per-head quantization scales and codes); it holds none of the
attention arithmetic. Both the fp64 oracle's tests and the HIP path's tests
and bench take their inputs from here.
"""

from .workloads import (  # noqa: F401
    Workload,
    Case,
    WORKLOADS,
    make_case,
    algorithmic_bytes,
    unit_subcase,
    WriteCase,
    make_write_case,
    visible_pairs,
    workload_lengths,
    workload_algorithmic_bytes,
    workload_visible_pairs,
)
