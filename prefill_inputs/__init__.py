"""Seeded synthetic prefill inputs (Q, K, V as bf16 bit patterns).

This package builds inputs only: random Gaussian activations with planted
attention structure.  It holds none of the sparse-attention method's
arithmetic, so both the fp64 oracle and the GPU path may draw from it.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    Shape,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    head_roles,
    make_inputs,
    workload,
    workload_inputs,
)
