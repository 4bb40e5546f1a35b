"""Seeded synthetic layer inputs shared by the oracle side and the HIP side.

This package holds workload descriptions and random draws only. It contains
none of the quantization method's arithmetic: the covariances, the incoherence
processing, the factorisation, the column sweep and the sensitivity score are
each implemented separately under ``oracle/`` and in the native library.
"""
from .gen import (  # noqa: F401
    BLOCK_BUDGET_BITS,
    BLOCK_WIDTHS,
    CHUNK,
    CONFIGS,
    WORKLOADS,
    LayerSpec,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    layer_specs,
    make_layer,
    make_signs,
    make_weights,
    token_chunk,
)
