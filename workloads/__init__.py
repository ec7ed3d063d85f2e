"""Seeded synthetic inputs for the verification step.

This package only draws random numbers and lays them out; it computes none of
the method (no union, probe, placement or attention).  Both the oracle-based
tests and the GPU path consume what it produces.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    StepInputs,
    History,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    make_history,
    make_step_inputs,
    make_hot_warm_set,
    make_resident_bitmaps,
    make_accepted,
    make_source_rows,
    positions_per_row,
    shrink,
)
