"""Seeded synthetic inputs for FFD decode attention.

This package only builds inputs (queries, bf16 K/V caches, sequence lengths)
and describes the benchmark workloads. It holds none of the method's
arithmetic: no quantiser, no scoring, no selection and no attention. Both the
CPU oracle and the HIP path consume what it produces.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    make_inputs,
    make_random_inputs,
    multi_query,
)
