"""Seeded synthetic inputs for the sparse-attention decode step.

This package draws raw inputs only: pre-RoPE queries and keys, values, the
low-rank projection matrices and planted "needle" keys.  It holds none of the
method's arithmetic (no RoPE, no indexer projection, no scoring, no top-p, no
attention); both the HIP library and the CPU oracle build their caches from
these draws with their own code.
"""
from .workload import (  # noqa: F401
    CONFIGS,
    Workload,
    WorkloadSpec,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_workload,
    spec_for,
)
