"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package only draws numbers and shapes them: it holds none of the
attention arithmetic, no window bookkeeping and no reference results.
"""
from .workloads import (
    WORKLOAD,
    WORKLOADS,
    Workload,
    TILE,
    draw_normal,
    draw_step_tensors,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    make_block_mask,
    diagonal_tiles,
)

__all__ = [
    "WORKLOAD",
    "WORKLOADS",
    "Workload",
    "TILE",
    "draw_normal",
    "draw_step_tensors",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_block_mask",
    "diagonal_tiles",
]
