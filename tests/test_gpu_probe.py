"""The measurement aids behind the bench's achievable peaks do the work they are timed for.

The MFMA loop's per-thread sums have a closed form (1024 * iters * bf16(value)^2, exact in
fp32 at these sizes), so every wave ran every MFMA step; the read probe's per-thread sums add
up to the sum of every 32-bit word of the buffer (mod 2^32), so every word was read exactly
once, including a tail that does not fill the grid."""

import numpy as np
import pytest
import torch

import mla_latent_kv_10_amd as mla

from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("iters,blocks,value", [(1, 1, 1.0), (1000, 8, 1.0), (777, 37, 0.5), (300, 1024, -2.0)])
def test_mfma_probe_sums(iters, blocks, value):
    say(f"mfma probe iters={iters} blocks={blocks} value={value}")
    sink = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    mla.probe_mfma_bf16(iters, blocks, value, sink)
    torch.cuda.synchronize()
    assert torch.all(sink.cpu() == 1024.0 * iters * value * value)


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (1 << 20, 3), ((1 << 22) + 48, 256), ((64 << 20) + 16, 1024)])
def test_read_probe_reads_every_word_once(nbytes, blocks):
    say(f"read probe bytes={nbytes} blocks={blocks}")
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-(2 ** 31), 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    src = host.to("cuda:0")
    sink = torch.full((blocks * 256,), -1, dtype=torch.int32, device="cuda:0")
    mla.probe_hbm_read(src, blocks, sink)
    torch.cuda.synchronize()
    got = int(sink.cpu().numpy().astype(np.uint32).astype(np.uint64).sum() % (1 << 32))
    want = int(host.numpy().astype(np.uint32).astype(np.uint64).sum() % (1 << 32))
    assert got == want
