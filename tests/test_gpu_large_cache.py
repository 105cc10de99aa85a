"""The largest caches the decode takes, and the FP8 writer past 4 GiB.

The decode addresses cache rows through buffer descriptors with 32-bit byte
offsets from the cache's start, so the host takes caches of at most 4 GiB
(larger ones are refused before any HIP call; the CPU tests check that).
Here the workload's pages are moved to the very top of a 4 GiB cache: the
output must equal the oracle's and, bit for bit, the same decode on the small
cache (the same metadata, so the same arithmetic order). The FP8 writer uses
64-bit addresses and is checked on rows past 4 GiB."""

import math

import numpy as np
import pytest
import torch

import mla_latent_kv_10_amd as mla
from oracle import quantize_rows
from workload import make_workload

from tests.gpu_helpers import compare, oracle, run_gpu, say, workload_floor_fn

pytestmark = pytest.mark.gpu

GIB4 = 1 << 32


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu()


@pytest.mark.parametrize("fmt,h_q,sparse", [("bf16", 128, False), ("bf16", 16, False), ("fp8", 128, False),
                                            ("fp8", 64, True), ("bf16", 128, True)])
def test_rows_at_the_top_of_a_4gib_cache(fmt, h_q, sparse):
    if sparse:
        w = make_workload(batch=2, s_q=1, h_q=h_q, kv_format=fmt, topk=300, sparse_tokens_per_seq=1024,
                          invalid_frac=0.05, seed=41)
    else:
        w = make_workload(batch=3, s_q=1, h_q=h_q, seqlens=[900, 130, 64], kv_format=fmt, seed=41)
    rb = w.kv.shape[2]
    total = GIB4 // (64 * rb)                 # the most pages a call takes
    base = total - w.num_blocks               # the workload's pages end at the last one
    say(f"4 GiB cache {fmt} h_q={h_q} sparse={sparse}: pages {base}..{total - 1} "
        f"(ending {total * 64 * rb / 2**30:.4f} GiB from the start)")
    small = run_gpu(w)
    torch.cuda.synchronize()
    dev = "cuda:0"
    big = torch.empty((total, 64, rb), dtype=torch.uint8, device=dev)
    big[base:] = w.kv.to(dev)
    g = {"q": w.q.to(dev), "kv": big, "cache_seqlens": w.cache_seqlens.to(dev)}
    if sparse:
        idx = w.indices.long()
        g["indices"] = torch.where(idx >= 0, idx + base * 64, idx).to(torch.int32).to(dev)
        g["block_table"] = None
    else:
        bt = w.block_table.long()
        g["block_table"] = torch.where(bt >= 0, bt + base, bt).to(torch.int32).to(dev)
        g["indices"] = None
    large = run_gpu(w, g)
    torch.cuda.synchronize()
    del big
    assert torch.equal(_bits(small[0]), _bits(large[0])) and torch.equal(_bits(small[1]), _bits(large[1]))
    o_ref, lse_ref = oracle(w)
    compare(large[0], large[1], o_ref, lse_ref, label=f"top of a 4 GiB cache ({fmt})", floor_fn=workload_floor_fn(w))


def test_fp8_writer_past_4gib():
    n = 300
    base_row = (math.ceil(GIB4 / 656) + 63) // 64 * 64 + 64
    say(f"fp8 writer past 4 GiB: rows from {base_row}")
    g = torch.Generator().manual_seed(42)
    src = torch.randn(n, 576, generator=g).to(torch.bfloat16)
    slots = (torch.randperm(2 * n, generator=g)[:n] + base_row).to(torch.int32)
    num_blocks = (base_row + 2 * n) // 64 + 1
    dev = "cuda:0"
    kv = torch.zeros((num_blocks, 64, 656), dtype=torch.uint8, device=dev)
    mla.quantize_fp8_append(src.to(dev), slots.to(dev), kv)
    torch.cuda.synchronize()
    got = kv.view(-1, 656)[slots.long().to(dev)].cpu().numpy()
    want = quantize_rows(src.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(got, want)
    # nothing landed below the slots (a 32-bit wrap would write near the start)
    assert int(kv.view(-1, 656)[:base_row].count_nonzero()) == 0
