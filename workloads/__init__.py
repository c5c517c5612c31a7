"""Seeded synthetic inputs for paged-KV attention.

This package is the one piece of code shared by the CPU oracle and the GPU
path.  It draws inputs only: page layouts, block tables, context lengths and
the q/K/V values.  It holds none of the attention arithmetic.
"""

from .gen import (  # noqa: F401
    Layout,
    WORKLOADS,
    bf16_bits_from_f32,
    decode_layout,
    cascade_layout,
    window_layout,
    mixed_layout,
    workload,
    values_numpy,
    values_torch,
    new_rows_numpy,
    new_rows_torch,
    pages_of,
    fp8_values_numpy,
    fp8_values_torch,
)
