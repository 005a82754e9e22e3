"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This package draws random numbers and lays them out; it performs no step of
the decode method itself (no scoring, selection, gathering or attention).
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    workload,
    make_layer,
    decode_step_inputs,
    layer_seed,
    request_lens,
    tie_scores,
    random_sorted_indices,
    bf16_bits,
    random_tensor,
    random_positions,
)
