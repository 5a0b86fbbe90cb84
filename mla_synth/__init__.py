"""Seeded synthetic inputs for the MLA decode step.

This package only draws random numbers, rounds them to the storage dtype and
lays out lengths and page tables.  It holds none of the attention arithmetic:
both the GPU library and the CPU oracle consume what it produces.
"""
from .workloads import (  # noqa: F401
    DSV2,
    LLAMA2_7B_MLA,
    Shape,
    TINY,
    Workload,
    WORKLOADS,
    workload,
    round_to_bf16,
    bf16_bits,
    bf16_bits_to_f32,
)
