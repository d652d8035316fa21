"""Seeded synthetic inputs for the multi-LoRA shrink/expand path.

This package only draws inputs (adapter maps, activations, adapter weights,
the output buffer's initial contents).  It holds none of the method's
arithmetic, so both the GPU path and the CPU oracle can consume what it makes.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    make_workload,
    make_integer_exact_workload,
    make_custom_workload,
    make_fuzz_mapping,
    make_mapping,
    workload_stats,
)
