"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This package only draws random tensors of the right shapes and distributions.
It holds none of the method's arithmetic (no hashing, no probabilities, no
selection, no attention), so both the GPU path and the CPU oracle can be fed
from it without sharing any computation.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    custom_workload,
    make_keys_values,
    make_query,
    make_hyperplanes,
    make_decode_inputs,
    planted_positions,
    seed_for,
)
