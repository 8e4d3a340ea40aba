"""Seeded synthetic inputs for paged decode attention.

This package only draws inputs: sequence lengths, block tables over a
shuffled page pool, and bf16 / fp8 value bit patterns.  It holds none of the
attention arithmetic, so both the fp64 oracle's tests and the HIP path's
tests and benchmark can take their inputs from it without sharing any of the
computation.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    GqaWorkload,
    MlaWorkload,
    bf16_bits_from_f32,
    fp8_codes_from_f32,
    gqa_workload,
    mla_workload,
)
