"""Seeded synthetic inputs for paged decode (shared by the oracle tests, the GPU
tests and the benchmark).

This package draws values and builds index arrays (block tables, context
lengths, slot mapping, copy pairs); it holds none of the attention arithmetic.
"""
from .generate import (  # noqa: F401
    Case,
    CONFIG_NAMES,
    MULTI_QUERY_NAMES,
    MultiQueryCase,
    bf16_bits_from_f32,
    draw_values,
    draw_e4m3_codes,
    Fp8Case,
    make_fp8_case,
    Int8Case,
    make_int8_case,
    make_aliased_case,
    make_case,
    make_fork_case,
    make_multi_query_case,
    make_multi_query_workload,
    make_prefix_case,
    make_private_case,
)
