"""Seeded synthetic inputs shared by the tests, the bench and the CPU oracle.

This package holds no arithmetic of the attention method itself: it only draws
random tensors, plants relevance structure, encodes values as bf16 bit patterns
and lays sequences out in memory.  Both the HIP path and the oracle consume what
it produces.
"""
from .gen import (  # noqa: F401
    Workload,
    bf16_bits_to_f32,
    extra_decode_queries,
    f32_to_bf16_bits,
    make_config,
    make_workload,
    upstream_grad,
    CONFIGS,
)
