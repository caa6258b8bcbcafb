"""Seeded synthetic inputs for the EntmaxKV decode step.

This module only draws random numbers and lays them out (bf16 rounding of
the generated fp32 values, page tables, sequence lengths).  It holds none of
the method's arithmetic, so both the CPU oracle and the HIP path can be fed
from it without sharing any computation.
"""
from .configs import (  # noqa: F401
    WorkloadSpec,
    CONFIG_NAMES,
    make_spec,
    queries,
    keys,
    values,
    page_table,
    seq_lens,
    round_to_bf16_bits,
)
