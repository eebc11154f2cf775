"""Seeded synthetic inputs shared by the oracle-side tests and the GPU side.

This package only draws numbers and names shapes.  It holds none of the
attention arithmetic: no scores, softmax, masks, slot mapping or rounding
points of the method.  Both the CPU oracle and the HIP path receive exactly
the arrays made here.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_to_f32,
    decode_inputs,
    prefill_inputs,
    randn_bf16_bits,
)
