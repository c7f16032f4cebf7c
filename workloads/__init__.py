"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package holds input construction and bf16 bit conversion only; it contains
none of the sparse-attention arithmetic.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_to_f32,
    bf16_bits_to_f64,
    f32_to_bf16_bits,
    get_workload,
    make_head,
    make_inputs,
    pos_code,
)
