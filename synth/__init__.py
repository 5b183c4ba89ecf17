"""Seeded synthetic inputs for the LSA indexer.

This package only draws random numbers and stores them in the key storage
dtype.  It contains no step of the indexer itself (no projection, clustering,
scoring or selection), so both the HIP path and the CPU oracle may use it.
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    gen_keys,
    gen_keys_head_f32,
    gen_keys_range,
    gen_positions,
    gen_queries,
    gen_W,
    get_workload,
)
