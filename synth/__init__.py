"""Seeded synthetic inputs for the NOSA decode-step hot path.

This package draws random numbers and nothing else: it holds none of the
method's arithmetic (no pooling, scoring, selection or attention). Both the
CPU oracle (through the tests) and the HIP path (through the tests and the
benchmark) take their inputs from here, so both see identical bf16 bits.
"""

from .workloads import (  # noqa: F401
    NEXT_WORKLOADS,
    WORKLOADS,
    Workload,
    bf16_bits_to_f32,
    bf16_bits_to_f64,
    context_kv,
    eviction_weights,
    f32_to_bf16_bits,
    f64_to_bf16_bits,
    forecasts,
    hot_blocks,
    new_tokens,
    queries,
    small_workload,
)
