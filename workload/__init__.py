"""Seeded synthetic inputs for MLA decode over a paged latent KV cache.

This package is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark. It draws random numbers, rounds them to bf16 and writes cache
rows in the byte layouts the decode reads; it holds none of the attention
arithmetic (no scores, softmax, masking or dequantisation).
"""

from .gen import (  # noqa: F401
    BLOCK_SIZE,
    D_QK,
    D_V,
    D_ROPE,
    ROW_BYTES,
    Workload,
    make_workload,
    config_workload,
    quantize_fp8_656,
    quantize_fp8_528,
    QK_DIMS,
    CONFIG_NAMES,
)
