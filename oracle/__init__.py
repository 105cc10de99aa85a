"""CPU oracle for MLA decode over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, float64 statement
of what the decode computes. Only the test suite, the smoke check in
``__graft_entry__`` and the benchmark's CPU-baseline leg may import it. The
GPU library and its Python binding never import, call or link it, and it
imports nothing from them.

Every function is pinned by tests that check it against facts fixed outside
this package (library routines, closed forms, invariants, page values); see
the ``tests/test_oracle_*.py`` files. No function here is "parity unpinned".
"""

from .mla_oracle import (  # noqa: F401
    E4M3FN_VALUES,
    FORMATS,
    ue8m0_values,
    bf16_bits_to_f64,
    f32_to_bf16_bits,
    decode_rows,
    attended_rows,
    attend,
    mla_decode_ref,
    lse_merge,
)
from .schedule import split_schedule, tile_counts  # noqa: F401
from .quantize import f32_to_e4m3fn_codes, quantize_rows, append_rows, quantize_rows_528  # noqa: F401
from .absorb import absorb_q, unabsorb_o  # noqa: F401
