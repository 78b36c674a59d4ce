"""Seeded synthetic inputs shaped like the GenRank workloads.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It only draws random numbers and lays them out; it holds none of the method's
arithmetic (no index derivation, no embedding sum, no attention, no bucketing).
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    Batch,
    Config,
    Tables,
    Weights,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_batch,
    make_config,
    make_labels,
    make_tables,
    make_weights,
    rt_boundaries,
)
