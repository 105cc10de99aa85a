"""Reference cache writer for the 656-byte FP8 row (quantise on write).

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the GPU path.

Pages cited (by title, then section):
  [Guide]       "FlashMLA 实战：MLA 注意力加速指南" (m.lsln.cn), sections
                "FP8 缓存怎么把 KV 压掉四成" (512 e4m3 codes, one fp32 scale per
                128 latent values, 64 RoPE values kept in bf16) and
                "容易踩的坑" (the writer must produce exactly this layout)
  [Walkthrough] "矩阵、注意力与 GPU：拆解 DeepGEMM 与 FlashMLA" (msy.plus),
                §三 (e4m3: 3 mantissa bits, largest finite value 448; one scale
                per block because a single scale would flush small values)

What is computed, for one 576-value bf16 row [latent 512 ; rope 64]:
  * for each group of 128 latent values: amax = max |x| (exact in fp32);
    scale = fp32(amax / 448), or 1 when amax is 0;
  * code = e4m3fn round-to-nearest-even of clamp(fp32(x / scale), -448, 448);
  * bytes [0, 512) codes, [512, 528) the four scales (little-endian fp32),
    [528, 656) the 64 rope values' bf16 bit patterns unchanged.

Readings where the pages are silent:
  * the scale is amax / 448 in fp32, both divisions are IEEE fp32 divisions
    rounded to nearest even, and the quotient is clamped before it is rounded
    to e4m3 (the pages give the format and the 448 maximum, not the quantiser);
  * a quotient that rounds to zero keeps its sign (code 0x80 for -0);
  * inputs are finite (NaN or infinite latent values are outside the writer's
    contract);
  * a row goes to absolute cache row ``slot = page * 64 + offset``, the same
    row numbering sparse indices use; slot -1, or any slot outside the cache,
    writes nothing; two rows aimed at one slot are outside the contract.
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import E4M3FN_VALUES

D_V = 512
D_ROPE = 64
GROUP = 128
FP8_MAX = np.float32(448.0)
ROW_BYTES = 656

# The non-negative finite e4m3fn values in code order: codes 0x00..0x7E are
# increasing in value (0, the seven subnormals, then the normals up to 448).
_POS_VALUES = E4M3FN_VALUES[:0x7F]
assert np.all(np.diff(_POS_VALUES) > 0)


def f32_to_e4m3fn_codes(y: np.ndarray) -> np.ndarray:
    """float32 values with |y| <= 448 -> e4m3fn codes, nearest value, ties to the even code.

    Nearest is decided exactly (float64 holds every float32 and every e4m3
    value); on a tie the code whose lowest mantissa bit is 0 wins. The sign
    bit is the sign bit of y, so -0 and negative values that round to 0 give
    0x80.
    """
    y = np.asarray(y, dtype=np.float32)
    if np.any(~np.isfinite(y)) or np.any(np.abs(y) > FP8_MAX):
        raise ValueError("f32_to_e4m3fn_codes takes finite values with |y| <= 448")
    a = np.abs(y).astype(np.float64)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << np.uint8(7)
    return code | sign


def quantize_rows(src_bf16_bits: np.ndarray) -> np.ndarray:
    """bf16 rows [n, 576] (uint16 bit patterns) -> 656-byte FP8 rows [n, 656] (uint8)."""
    bits = np.asarray(src_bf16_bits, dtype=np.uint16)
    if bits.ndim != 2 or bits.shape[1] != D_V + D_ROPE:
        raise ValueError("quantize_rows takes bf16 rows of 576 values")
    n = bits.shape[0]
    latent = (bits[:, :D_V].astype(np.uint32) << np.uint32(16)).view(np.float32)  # exact bf16 -> fp32
    groups = latent.reshape(n, D_V // GROUP, GROUP)
    if not np.all(np.isfinite(groups)):
        raise ValueError("quantize_rows takes finite latent values")
    amax = np.abs(groups).max(axis=2)                          # float32, exact
    with np.errstate(under="ignore"):
        scale = np.where(amax == 0, np.float32(1.0), amax / FP8_MAX).astype(np.float32)
        y = (groups / scale[:, :, None]).astype(np.float32)    # fp32 IEEE division
    y = np.clip(y, -FP8_MAX, FP8_MAX)
    codes = f32_to_e4m3fn_codes(y).reshape(n, D_V)
    out = np.empty((n, ROW_BYTES), dtype=np.uint8)
    out[:, :D_V] = codes
    out[:, D_V:D_V + 16] = scale.astype("<f4").view(np.uint8).reshape(n, 16)
    out[:, D_V + 16:] = bits[:, D_V:].astype("<u2").view(np.uint8).reshape(n, 2 * D_ROPE)
    return out


def append_rows(cache_rows: np.ndarray, slots: np.ndarray, src_bf16_bits: np.ndarray) -> np.ndarray:
    """Copy of ``cache_rows`` [num_rows, 656] with quantised source row i written at row slots[i].

    Slots outside [0, num_rows) (including -1) write nothing.
    """
    out = np.array(cache_rows, dtype=np.uint8, copy=True)
    rows = quantize_rows(src_bf16_bits)
    slots = np.asarray(slots, dtype=np.int64)
    ok = (slots >= 0) & (slots < out.shape[0])
    out[slots[ok]] = rows[ok]
    return out


# --------------------------------------------------------------------------
# The 528-byte row: 512 e4m3 codes + 16 UE8M0 scales
# --------------------------------------------------------------------------
#
# [Walkthrough] §八 (the V4.1 format: 528 bytes per token, 512 FP8 values and
# 16 UE8M0 scales, RoPE quantised too), §九 (data first, scales after) and §三
# (a UE8M0 scale is a power of two with no mantissa, rounded *up* to a power
# of two). Readings where the pages are silent:
#   * the 512 values are the whole key row, 448 latent dims then 64 RoPE
#     dims; scale j covers values 32 j .. 32 j + 31 (16 blocks of 32);
#   * the scale of a block is the smallest power of two 2^k with
#     448 * 2^k >= amax (2^0 for an all-zero block); its byte is k + 127,
#     at least 0;
#   * code = e4m3fn round-to-nearest-even of x / 2^k (exact division, at most
#     448 in magnitude, so no clamp); signed zeros as for the 656-byte row.

ROW_528 = 528
D_528 = 512
MX_BLOCK = 32


def ue8m0_exponent_for(amax: np.ndarray) -> np.ndarray:
    """Smallest k with 448 * 2^k >= amax, for amax > 0 (float32 values, exact).

    With amax = f * 2^E, f in [0.5, 1) (frexp) and 448 = 0.875 * 2^9:
    448 * 2^k >= amax  <=>  k >= E - 9 when f <= 0.875, else k >= E - 8.
    """
    f, E = np.frexp(np.asarray(amax, dtype=np.float64))
    return (E - 9 + (f > 0.875)).astype(np.int64)


def quantize_rows_528(src_bf16_bits: np.ndarray) -> np.ndarray:
    """bf16 key rows [n, 512] (uint16 bit patterns: 448 latent, 64 RoPE) -> 528-byte rows [n, 528]."""
    bits = np.asarray(src_bf16_bits, dtype=np.uint16)
    if bits.ndim != 2 or bits.shape[1] != D_528:
        raise ValueError("quantize_rows_528 takes bf16 rows of 512 values")
    n = bits.shape[0]
    x = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).reshape(n, D_528 // MX_BLOCK, MX_BLOCK)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_rows_528 takes finite values")
    amax = np.abs(x).max(axis=2)
    k = np.where(amax == 0, 0, ue8m0_exponent_for(np.where(amax == 0, 1.0, amax)))
    e = np.maximum(k + 127, 0)
    k = e - 127
    y = np.ldexp(x.astype(np.float64), -k[:, :, None])      # exact: a power-of-two scaling
    codes = f32_to_e4m3fn_codes(y.astype(np.float32)).reshape(n, D_528)
    out = np.empty((n, ROW_528), dtype=np.uint8)
    out[:, :D_528] = codes
    out[:, D_528:] = e.astype(np.uint8)
    return out
