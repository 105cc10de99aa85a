"""Seeded synthetic workloads with the shapes of the pages' decode workloads.

Page keys used in citations:
  "FlashMLA 实战：MLA 注意力加速指南" (m.lsln.cn) -- the FlashMLA usage guide
  "矩阵、注意力与 GPU：拆解 DeepGEMM 与 FlashMLA" (msy.plus) -- the DeepGEMM/FlashMLA walkthrough

Layouts written here:
  * bf16 cache row: 576 bf16 values = 512 latent dims then 64 RoPE dims,
    1152 bytes, tokens contiguous inside a 64-token page
    (walkthrough §六 "位置编码必须解耦" orders the key as [latent; rope];
    usage guide §"FP8 缓存怎么把 KV 压掉四成" gives 1152 B per bf16 token).
  * FP8 cache row, 656 bytes: 512 e4m3 codes, then 4 little-endian fp32
    scales (one per 128 latent dims), then 64 bf16 RoPE values
    (usage guide §"FP8 缓存..." and §"容易踩的坑"; walkthrough §八 format list).

Random draws happen in a fixed order per workload: sequence lengths, q,
cache contents, page permutation, sparse indices, positions set to -1.
All draws use one CPU ``torch.Generator`` seeded with ``seed``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np
import torch

BLOCK_SIZE = 64  # tokens per KV page (walkthrough §七 version table: paged KV, block 64)
D_QK = 576
D_V = 512
D_ROPE = 64
ROW_BYTES = {"bf16": 1152, "fp8": 656, "fp8_528": 528}
QK_DIMS = {"bf16": 576, "fp8": 576, "fp8_528": 512}   # key (and query) dims per format
FP8_GROUP = 128
FP8_MAX = 448.0  # largest finite e4m3 magnitude (walkthrough §三 "为什么要量化")

CONFIG_NAMES = {
    1: "tiny dense bf16: B=1 s_q=1 h_q=4 L=256",
    2: "dense bf16: B=16 s_q=1 h_q=128 L~U[1024,4096]",
    3: "low-head dense bf16: B=16 s_q=1 h_q=16 L fixed",
    4: "fp8 paged causal: B=64 s_q=2 h_q=128 L=8192",
    5: "sparse fp8: B=32 s_q=1 h_q=128 topk=2048 (5% -1)",
    6: "sparse prefill bf16: B=1 s_q=1024 h_q=128 topk=2048 over a 32768-token prefix",
    7: "dense bf16 64-head share: B=16 s_q=1 h_q=64 L~U[1024,4096]",
    8: "fp8_528 paged causal: B=64 s_q=2 h_q=128 L=8192",
    9: "sparse fp8_528: B=32 s_q=1 h_q=128 topk=2048 (5% -1)",
    10: "low-head two-position causal bf16: B=16 s_q=2 h_q=16 L=65536",
}


@dataclass
class Workload:
    """One decode call's inputs, all on the CPU.

    q            bf16 [B, s_q, h_q, 576]
    kv           uint8 [num_blocks, 64, row_bytes]  (bf16 rows viewed as bytes, or 656-B FP8 rows)
    kv_format    "bf16" or "fp8"
    block_table  int32 [B, max_blocks_per_seq] or None (sparse)
    cache_seqlens int32 [B]
    indices      int32 [B, s_q, topk] or None (dense); -1 marks an unused slot
    """

    name: str
    q: torch.Tensor
    kv: torch.Tensor
    kv_format: str
    block_table: Optional[torch.Tensor]
    cache_seqlens: torch.Tensor
    indices: Optional[torch.Tensor]
    softmax_scale: float
    causal: bool
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def s_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def h_q(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_blocks(self) -> int:
        return int(self.kv.shape[0])

    @property
    def topk(self) -> int:
        return 0 if self.indices is None else int(self.indices.shape[2])


def _normal_bf16(gen: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def quantize_fp8_656(latent: torch.Tensor, rope_bf16: torch.Tensor) -> torch.Tensor:
    """Cache writer: fp32 latent [N, 512] + bf16 rope [N, 64] -> uint8 rows [N, 656].

    Per group of 128 latent values: scale = fp32(amax / 448) (scale 1 when the
    group is all zero); code = e4m3 round-to-nearest-even of clamp(x / scale,
    +-448), computed in fp32. The clamp comes first because torch's e4m3fn cast
    maps magnitudes above the largest finite code to NaN.
    """
    assert latent.dtype == torch.float32 and latent.shape[1] == D_V
    assert rope_bf16.dtype == torch.bfloat16 and rope_bf16.shape[1] == D_ROPE
    n = latent.shape[0]
    groups = latent.reshape(n, D_V // FP8_GROUP, FP8_GROUP)
    amax = groups.abs().amax(dim=2)
    scale = (amax / FP8_MAX).to(torch.float32)
    scale = torch.where(amax == 0, torch.ones_like(scale), scale)
    scaled = (groups / scale.unsqueeze(2)).clamp(-FP8_MAX, FP8_MAX)
    codes = scaled.to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, D_V)
    out = torch.empty((n, ROW_BYTES["fp8"]), dtype=torch.uint8)
    out[:, :512] = codes
    out[:, 512:528] = scale.contiguous().view(torch.uint8).reshape(n, 16)
    out[:, 528:656] = rope_bf16.contiguous().view(torch.uint8).reshape(n, 128)
    return out


def quantize_fp8_528(x: torch.Tensor) -> torch.Tensor:
    """Cache writer for the 528-byte row: fp32 key rows [N, 512] (448 latent,
    then 64 RoPE) -> uint8 rows [N, 528].

    Per block of 32 values: the scale is the smallest power of two 2^k with
    448 * 2^k >= amax (2^0 for an all-zero block), stored as the byte k + 127
    (UE8M0: walkthrough §三, scales rounded up to a power of two); code = e4m3
    round-to-nearest-even of x / 2^k (exact; |x / 2^k| <= 448). Codes first,
    the 16 scale bytes after (walkthrough §八, §九).
    """
    assert x.dtype == torch.float32 and x.shape[1] == 512
    n = x.shape[0]
    blocks = x.reshape(n, 16, 32)
    amax = blocks.abs().amax(dim=2).to(torch.float64)
    k = torch.zeros_like(amax, dtype=torch.int64)
    nz = amax > 0
    # smallest k with 448 * 2^k >= amax, searched from log2 and corrected exactly
    k[nz] = torch.ceil(torch.log2(amax[nz] / 448.0)).to(torch.int64)
    k[nz] += (torch.ldexp(torch.full_like(amax[nz], 448.0), k[nz]) < amax[nz]).to(torch.int64)
    k[nz] -= (torch.ldexp(torch.full_like(amax[nz], 448.0), k[nz] - 1) >= amax[nz]).to(torch.int64)
    e = torch.clamp(k + 127, min=0)
    k = e - 127
    y = torch.ldexp(blocks.to(torch.float64), -k.unsqueeze(2)).to(torch.float32)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, 512)
    out = torch.empty((n, 528), dtype=torch.uint8)
    out[:, :512] = codes
    out[:, 512:] = e.to(torch.uint8)
    return out


def _cache_rows(gen: torch.Generator, n_rows: int, kv_format: str, chunk: int = 1 << 16) -> torch.Tensor:
    """n_rows cache rows drawn from N(0,1), in the requested byte layout (chunked to bound memory)."""
    rb = ROW_BYTES[kv_format]
    out = torch.empty((n_rows, rb), dtype=torch.uint8)
    for s in range(0, n_rows, chunk):
        e = min(n_rows, s + chunk)
        if kv_format == "bf16":
            out[s:e] = _normal_bf16(gen, (e - s, D_QK)).view(torch.uint8).reshape(e - s, rb)
        elif kv_format == "fp8_528":
            out[s:e] = quantize_fp8_528(torch.randn(e - s, 512, generator=gen, dtype=torch.float32))
        else:
            latent = torch.randn(e - s, D_V, generator=gen, dtype=torch.float32)
            rope = _normal_bf16(gen, (e - s, D_ROPE))
            out[s:e] = quantize_fp8_656(latent, rope)
    return out


def make_workload(
    *,
    batch: int,
    s_q: int,
    h_q: int,
    seqlens: Optional[Sequence[int]] = None,
    seqlen_range: Optional[tuple] = None,
    kv_format: str = "bf16",
    causal: bool = False,
    topk: int = 0,
    sparse_tokens_per_seq: int = 0,
    invalid_frac: float = 0.0,
    prefix_sparse: bool = False,
    shuffle_pages: bool = True,
    extra_blocks: int = 0,
    softmax_scale: Optional[float] = None,
    seed: int = 0,
    name: str = "custom",
) -> Workload:
    """Build a workload.

    Dense (topk == 0): sequence b holds seqlens[b] tokens in ceil(L/64) pages
    drawn from a pool of sum(ceil(L/64)) + extra_blocks pages; the pool order
    is a random permutation when shuffle_pages. block_table entries past a
    sequence's last page are -1.

    Sparse (topk > 0): the cache is contiguous, sequence b owning rows
    [b*T, (b+1)*T) with T = sparse_tokens_per_seq; indices[b, i, :] are topk
    distinct rows of that range in random order; round(invalid_frac * topk)
    positions per (b, i) are set to -1. block_table is None and cache_seqlens
    holds T. With prefix_sparse (a prefill chunk: the s_q queries are the
    sequence's last s_q tokens), query i at position T - s_q + i draws its
    topk rows from its own visible prefix [0, T - s_q + i] instead.
    """
    gen = torch.Generator().manual_seed(seed)
    if softmax_scale is None:
        softmax_scale = float(np.float32(D_QK ** -0.5))
    meta: dict = {"seed": seed}
    if topk == 0:
        if seqlens is None:
            lo, hi = seqlen_range
            seqlens_t = torch.randint(lo, hi + 1, (batch,), generator=gen, dtype=torch.int64)
        else:
            seqlens_t = torch.tensor(list(seqlens), dtype=torch.int64)
        assert seqlens_t.numel() == batch
        q = _normal_bf16(gen, (batch, s_q, h_q, QK_DIMS[kv_format]))
        pages = [int(math.ceil(int(l) / BLOCK_SIZE)) for l in seqlens_t.tolist()]
        pool = sum(pages) + extra_blocks
        pool = max(pool, 1)
        kv = _cache_rows(gen, pool * BLOCK_SIZE, kv_format).reshape(pool, BLOCK_SIZE, ROW_BYTES[kv_format])
        perm = torch.randperm(pool, generator=gen) if shuffle_pages else torch.arange(pool)
        max_pages = max(max(pages), 1)
        bt = torch.full((batch, max_pages), -1, dtype=torch.int32)
        off = 0
        for b, n in enumerate(pages):
            bt[b, :n] = perm[off:off + n].to(torch.int32)
            off += n
        return Workload(name, q, kv, kv_format, bt, seqlens_t.to(torch.int32), None,
                        softmax_scale, causal, meta)
    # sparse
    T = sparse_tokens_per_seq
    assert T % BLOCK_SIZE == 0 and topk <= T and not causal
    q = _normal_bf16(gen, (batch, s_q, h_q, QK_DIMS[kv_format]))
    n_blocks = batch * T // BLOCK_SIZE
    kv = _cache_rows(gen, n_blocks * BLOCK_SIZE, kv_format).reshape(n_blocks, BLOCK_SIZE, ROW_BYTES[kv_format])
    idx = torch.empty((batch, s_q, topk), dtype=torch.int32)
    for b in range(batch):
        for i in range(s_q):
            visible = T - s_q + i + 1 if prefix_sparse else T
            assert visible >= topk
            idx[b, i] = (torch.randperm(visible, generator=gen)[:topk] + b * T).to(torch.int32)
    n_inv = int(round(invalid_frac * topk))
    if n_inv:
        for b in range(batch):
            for i in range(s_q):
                pos = torch.randperm(topk, generator=gen)[:n_inv]
                idx[b, i, pos] = -1
    seqlens_t = torch.full((batch,), T, dtype=torch.int32)
    meta["invalid_per_row"] = n_inv
    return Workload(name, q, kv, kv_format, None, seqlens_t, idx, softmax_scale, False, meta)


def config_workload(cfg: int, seqlen: int = 8192, seed: int = 0) -> Workload:
    """The five decode workloads, the sparse prefill chunk (6), the 64-head share (7), the two FP8 shapes
    with 528-byte rows (8, 9) and the two-position low-head share (10); config 3 takes its fixed sequence
    length."""
    if cfg == 1:
        # q and cache drawn in fp32 then rounded to bf16; 4 pages, shuffled.
        return make_workload(batch=1, s_q=1, h_q=4, seqlens=[256], kv_format="bf16",
                             seed=seed, name=CONFIG_NAMES[1])
    if cfg == 2:
        return make_workload(batch=16, s_q=1, h_q=128, seqlen_range=(1024, 4096), kv_format="bf16",
                             seed=seed, name=CONFIG_NAMES[2])
    if cfg == 3:
        return make_workload(batch=16, s_q=1, h_q=16, seqlens=[seqlen] * 16, kv_format="bf16",
                             seed=seed, name=CONFIG_NAMES[3] + f" L={seqlen}")
    if cfg == 4:
        return make_workload(batch=64, s_q=2, h_q=128, seqlens=[8192] * 64, kv_format="fp8",
                             causal=True, seed=seed, name=CONFIG_NAMES[4])
    if cfg == 5:
        return make_workload(batch=32, s_q=1, h_q=128, kv_format="fp8", topk=2048,
                             sparse_tokens_per_seq=32768, invalid_frac=0.05, seed=seed,
                             name=CONFIG_NAMES[5])
    if cfg == 6:
        return make_workload(batch=1, s_q=1024, h_q=128, kv_format="bf16", topk=2048,
                             sparse_tokens_per_seq=32768, prefix_sparse=True, seed=seed, name=CONFIG_NAMES[6])
    if cfg == 7:
        # one GPU's share of 128 heads under two-way head sharding: the dense
        # bf16 lengths with 64 heads (the 64-head row-group kernel)
        return make_workload(batch=16, s_q=1, h_q=64, seqlen_range=(1024, 4096), kv_format="bf16",
                             seed=seed, name=CONFIG_NAMES[7])
    if cfg == 8:
        # the FP8 causal shape with 528-byte rows (512 e4m3 codes, 16 UE8M0 scales)
        return make_workload(batch=64, s_q=2, h_q=128, seqlens=[8192] * 64, kv_format="fp8_528",
                             causal=True, seed=seed, name=CONFIG_NAMES[8])
    if cfg == 9:
        # the sparse FP8 shape with 528-byte rows
        return make_workload(batch=32, s_q=1, h_q=128, kv_format="fp8_528", topk=2048,
                             sparse_tokens_per_seq=32768, invalid_frac=0.05, seed=seed, name=CONFIG_NAMES[9])
    if cfg == 10:
        # the low-head share with two query positions per sequence (a draft
        # token verified with the next one): 32 rows attend one cache
        return make_workload(batch=16, s_q=2, h_q=16, seqlens=[65536] * 16, kv_format="bf16",
                             causal=True, seed=seed, name=CONFIG_NAMES[10])
    raise ValueError(f"unknown config {cfg}")
