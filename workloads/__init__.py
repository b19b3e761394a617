"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This package only draws random numbers and rounds them to the storage types the
path consumes (bf16 activations/weights, fp32 factors and clip logits).  It holds
none of the method's arithmetic: no transform, no clipping, no quantisation.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    SWEEP_A,
    Workload,
    bf16_bits_to_f32,
    f64_to_bf16_bits,
    make_workload,
)
