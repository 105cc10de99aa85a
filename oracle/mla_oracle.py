"""Float64 reference for absorbed-MLA decode attention over a paged latent cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the GPU path.

Pages cited (by title, then section):
  [Walkthrough] "矩阵、注意力与 GPU：拆解 DeepGEMM 与 FlashMLA" (msy.plus)
  [Guide]       "FlashMLA 实战：MLA 注意力加速指南" (m.lsln.cn)

What is computed (for every batch b, query position i < s_q, head h):
  * Absorbed MLA is MQA: every head scores against the same 576-dim cache row
    [latent c (512) ; rope k^R (64)] and the value is the 512-dim latent itself
    ([Walkthrough] §六 "吸收" and "结果：decode 变成 MQA").
  * Attention is the naive definition: explicit score vector, then a two-pass
    softmax (max, then exponentials and their sum), then the weighted sum of
    values ([Walkthrough] §五 "公式" and the naive attention listing that
    keeps S materialised).
  * lse is the natural log of the sum of exp(score) over attended tokens.

Readings where the pages are silent:
  * causal alignment is bottom-right: query i sees cache positions
    t <= L - s_q + i;
  * an empty attended set gives o = 0 and lse = -inf;
  * a sparse index outside [0, num_rows) is treated like -1 (skipped);
    duplicate indices each count;
  * a dense position whose page id is not a cache page (e.g. -1), or past
    the block table's row, is skipped in the same way;
  * FP8 rows dequantise as bf16_rne(fp32(code) * fp32(scale)), the product
    rounded once to fp32, then once to bf16.
  * the 528-byte row ([Walkthrough] §八, the V4.1 format: 512 FP8 values and
    16 UE8M0 scales, RoPE quantised too, data before scales; §十 lists
    528 = 512 fp8 + 16 ue8m0) holds the whole 512-dim key: 448 latent dims,
    then the 64 RoPE dims the other formats carry, so d_qk = 512 and the
    value is the 448-dim latent; scale j (a byte e, value 2^(e - 127), 255 is
    NaN) applies to values 32 j .. 32 j + 31, the block size that gives 16
    scales for 512 values.
"""

from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np

BLOCK_SIZE = 64
D_QK = 576
D_V = 512

# Row formats: bytes per cached token, key dims (d_qk), value dims (d_v).
FORMATS = {
    "bf16": (1152, 576, 512),
    "fp8": (656, 576, 512),
    "fp8_528": (528, 512, 448),
}
MX_BLOCK = 32   # values per UE8M0 scale in the 528-byte row


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def _e4m3fn_value(code: int) -> float:
    """OCP FP8 E4M3 ("fn": no infinities) decoded from its definition.

    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits. Exponent 0 is
    subnormal (m/8 * 2^-6); S.1111.111 is NaN; the largest finite value is
    1.75 * 2^8 = 448 ([Walkthrough] §三 gives e4m3's maximum as 448).
    """
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (-6)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


E4M3FN_VALUES = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even. NaN stays NaN."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    quiet_nan = ((u >> 16) | 0x0040) & 0xFFFF
    return np.where(is_nan, quiet_nan, rounded).astype(np.uint16)


# --------------------------------------------------------------------------
# Cache rows
# --------------------------------------------------------------------------

def ue8m0_values(e: np.ndarray) -> np.ndarray:
    """UE8M0 scale bytes -> their values 2^(e - 127) as float32 (255 is NaN).

    [Walkthrough] §三 (scale layout): a UE8M0 scale stores only a power of
    two, an 8-bit exponent with no mantissa. e = 0 gives 2^-127, a float32
    subnormal, still exact.
    """
    e = np.asarray(e, dtype=np.int64)
    with np.errstate(over="ignore"):
        v = np.ldexp(np.float64(1.0), e - 127).astype(np.float32)
    return np.where(e == 255, np.float32(np.nan), v)


def decode_rows(rows: np.ndarray, kv_format: str) -> np.ndarray:
    """Raw cache rows (uint8 [n, row_bytes]) -> exact float64 values [n, d_qk].

    bf16 rows: 576 little-endian bf16 values (512 latent, then 64 rope).
    fp8 rows ([Guide] §"FP8 缓存怎么把 KV 压掉四成", §"容易踩的坑"): bytes
    [0, 512) are e4m3 codes for the latent, [512, 528) four little-endian fp32
    scales, one per 128 latent dims, [528, 656) the 64 rope values as bf16.
    fp8_528 rows ([Walkthrough] §八, §九 "数据在前、scale 在后"): bytes
    [0, 512) are e4m3 codes of all 512 key dims (448 latent, 64 rope), bytes
    [512, 528) sixteen UE8M0 scales, scale j for dims 32 j .. 32 j + 31;
    value = bf16_rne(fp32(code) * 2^(e - 127)), exact unless it leaves the
    range of bf16.
    """
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    n = rows.shape[0]
    if kv_format == "fp8_528":
        assert rows.shape[1] == 528
        code_vals = E4M3FN_VALUES[rows[:, :512]].astype(np.float32)
        block_scale = np.repeat(ue8m0_values(rows[:, 512:528]), MX_BLOCK, axis=1)
        with np.errstate(invalid="ignore", over="ignore", under="ignore"):
            prod = code_vals * block_scale  # one fp32 rounding (exact within range)
        return bf16_bits_to_f64(f32_to_bf16_bits(prod))
    if kv_format == "bf16":
        assert rows.shape[1] == 1152
        return bf16_bits_to_f64(rows.view("<u2").reshape(n, D_QK))
    assert kv_format == "fp8" and rows.shape[1] == 656
    codes = rows[:, :512]
    scales = rows[:, 512:528].copy().view("<f4").reshape(n, 4)
    rope_bits = rows[:, 528:656].copy().view("<u2").reshape(n, 64)
    code_vals = E4M3FN_VALUES[codes].astype(np.float32)  # exact: e4m3 values fit fp32
    group_scale = np.repeat(scales, 128, axis=1).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        prod = code_vals * group_scale  # one fp32 rounding
    latent = bf16_bits_to_f64(f32_to_bf16_bits(prod))
    out = np.empty((n, D_QK), dtype=np.float64)
    out[:, :512] = latent
    out[:, 512:] = bf16_bits_to_f64(rope_bits)
    return out


def attended_rows(
    b: int,
    i: int,
    *,
    s_q: int,
    num_rows: int,
    block_table: Optional[np.ndarray],
    cache_seqlens: Optional[np.ndarray],
    causal: bool,
    indices: Optional[np.ndarray],
) -> np.ndarray:
    """Cache row ids attended by query (b, i), in order (a multiset for sparse).

    Dense: positions t < L_b (causal: t <= L_b - s_q + i); position t lives in
    page block_table[b, t // 64] at offset t % 64, i.e. row page*64 + t%64.
    A position whose page id is not a page of the cache (outside
    [0, num_rows / 64), e.g. -1) or that lies past the block table's row
    (t >= 64 * max_blocks_per_seq) has no cache row and is skipped: the pages
    never say what such a slot holds, so it is read as absent.
    Sparse ([Walkthrough] §八 "当前 master 已经是稀疏注意力"; [Guide]
    §"怎么用起来"): the listed absolute rows page*block_size + offset; -1
    entries are skipped, and so is anything outside [0, num_rows).
    """
    if indices is not None:
        idx = np.asarray(indices[b, i], dtype=np.int64)
        return idx[(idx >= 0) & (idx < num_rows)]
    L = int(cache_seqlens[b])
    limit = L - s_q + 1 + i if causal else L
    limit = max(0, min(limit, L))
    table = np.asarray(block_table[b], dtype=np.int64)
    limit = min(limit, table.shape[0] * BLOCK_SIZE)
    t = np.arange(limit, dtype=np.int64)
    pages = table[t // BLOCK_SIZE]
    keep = (pages >= 0) & (pages < num_rows // BLOCK_SIZE)
    return pages[keep] * BLOCK_SIZE + t[keep] % BLOCK_SIZE


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def attend(q: np.ndarray, K: np.ndarray, scale: float, d_v: int = D_V) -> Tuple[np.ndarray, np.ndarray]:
    """Naive attention of h query rows against n keys; V = K[:, :d_v] (the latent).

    q: [h, d_qk] float64, K: [n, d_qk] float64. Returns o [h, d_v], lse [h].
    Scores are formed explicitly, then a two-pass softmax.
    """
    h = q.shape[0]
    n = K.shape[0]
    if n == 0:
        return np.zeros((h, d_v)), np.full(h, -np.inf)
    S = (q @ K.T) * scale                      # [h, n] explicit score matrix
    m = S.max(axis=1, keepdims=True)           # pass 1: row max
    E = np.exp(S - m)                          # pass 2: exponentials
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    o = P @ K[:, :d_v]
    lse = (m + np.log(l))[:, 0]
    return o, lse


def mla_decode_ref(
    q: np.ndarray,
    kv: np.ndarray,
    kv_format: str,
    *,
    block_table: Optional[np.ndarray],
    cache_seqlens: Optional[np.ndarray],
    softmax_scale: float,
    causal: bool = False,
    indices: Optional[np.ndarray] = None,
    rows: Optional[Iterable[Tuple[int, int]]] = None,
    kv_is_decoded: bool = False,
) -> Tuple[np.ndarray, np.ndarray]:
    """Reference decode.

    q: bf16 bit patterns uint16 [B, s_q, h_q, d_qk] (or float64 values).
    kv: uint8 [num_blocks, 64, row_bytes] raw cache, or float64
        [num_blocks*64, d_qk] already-decoded rows when kv_is_decoded.
    kv_format: "bf16", "fp8" (d_qk 576, d_v 512) or "fp8_528" (d_qk 512,
        d_v 448); with kv_is_decoded, d_v is 512 when d_qk is 576, else 448.
    softmax_scale is used as the float64 value of its float32 rounding.
    rows: optional subset of (b, i) pairs to evaluate (others left NaN).
    Returns o float64 [B, s_q, h_q, d_v] and lse float64 [B, s_q, h_q].
    """
    q = np.asarray(q)
    qv = bf16_bits_to_f64(q) if q.dtype == np.uint16 else q.astype(np.float64)
    B, s_q, h_q, _ = qv.shape
    if kv_is_decoded:
        num_rows = kv.shape[0]
    else:
        num_rows = kv.shape[0] * kv.shape[1]
        flat = kv.reshape(num_rows, kv.shape[2])
    scale = float(np.float32(softmax_scale))
    if causal and indices is not None:
        raise ValueError("causal masking is defined for dense attention only")
    d_qk = qv.shape[3]
    d_v = FORMATS[kv_format][2] if not kv_is_decoded else (D_V if d_qk == D_QK else 448)
    if not kv_is_decoded and d_qk != FORMATS[kv_format][1]:
        raise ValueError(f"q has {d_qk} dims; a {kv_format} cache row has {FORMATS[kv_format][1]}")
    o = np.full((B, s_q, h_q, d_v), np.nan)
    lse = np.full((B, s_q, h_q), np.nan)
    pairs = rows if rows is not None else [(b, i) for b in range(B) for i in range(s_q)]
    for b, i in pairs:
        r = attended_rows(b, i, s_q=s_q, num_rows=num_rows, block_table=block_table,
                          cache_seqlens=cache_seqlens, causal=causal, indices=indices)
        K = kv[r] if kv_is_decoded else decode_rows(flat[r], kv_format)
        o[b, i], lse[b, i] = attend(qv[b, i], K, scale, d_v)
    return o, lse


def lse_merge(os_: np.ndarray, lses: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Merge attention over disjoint key sets from their normalised partials.

    os_: [k, ..., 512] each partial's softmax-weighted output; lses: [k, ...].
    The split merge of [Walkthrough] §七 "split-KV：把长序列切开": with running
    maxima m_j and sums l_j, m = max m_j, l = sum l_j e^{m_j - m},
    o = sum o_j l_j e^{m_j - m} / l. With lse_j = m_j + ln l_j this is
    o = sum_j e^{lse_j - lse} o_j and lse = ln sum_j e^{lse_j}. Partials with
    lse = -inf (empty key sets) weigh zero; all empty gives o = 0, lse = -inf.
    """
    os_ = np.asarray(os_, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - m_safe), 0.0)
    l = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    wn = np.where(l > 0, w / np.where(l > 0, l, 1.0), 0.0)
    o = (wn[..., None] * np.where(np.isfinite(lses)[..., None], os_, 0.0)).sum(axis=0)
    return o, lse
