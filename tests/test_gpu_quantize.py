"""FP8 cache writer on the GPU (mla_quantize_fp8_append through the C ABI) against
the oracle's writer, byte for byte: the codes, scales and RoPE bytes are integer
results, so the bar is bit-exact."""

import numpy as np
import pytest
import torch

import mla_latent_kv_10_amd as mla
from oracle import append_rows, mla_decode_ref, quantize_rows

from tests.gpu_helpers import compare, say, workload_floor_fn
from workload.gen import Workload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bits(x: torch.Tensor) -> np.ndarray:
    return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _gpu_write(src_bits: np.ndarray, slots: np.ndarray, cache: np.ndarray) -> np.ndarray:
    """Run the writer on the GPU: src bf16 bits [n, 576], slots [n], cache bytes [num_rows, 656]."""
    num_rows = cache.shape[0]
    src = torch.from_numpy(src_bits.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    sl = torch.from_numpy(slots.astype(np.int32)).to(DEV)
    kv = torch.from_numpy(cache.copy()).to(DEV).view(num_rows // 64, 64, 656)
    mla.quantize_fp8_append(src, sl, kv)
    torch.cuda.synchronize()
    return kv.view(num_rows, 656).cpu().numpy()


def _random_rows(n: int, seed: int) -> np.ndarray:
    g = torch.Generator().manual_seed(seed)
    mag = torch.exp(3 * torch.randn(n, 4, generator=g)).repeat_interleave(128, 1)
    latent = (torch.randn(n, 512, generator=g) * mag).to(torch.bfloat16)
    latent[0, :128] = 0                                   # all-zero group: scale 1
    latent[1, 128:256] = -latent[1, 128:256].abs()        # negative-only group
    latent[2, 256:384] *= 1e-30                            # tiny group (scale far below 1)
    latent[3, 384:512] = latent[3, 384:512] * 1e30         # huge group
    latent[4, :] = 0
    latent[4, 5] = -448                                    # amax from a negative value
    latent[5, 130] = 3e38                                  # near the top of bf16's range
    latent[6, 256:384] = (torch.randn(128, generator=g) * 1e-38).to(torch.bfloat16)  # subnormal values, subnormal scale
    rope = torch.randn(n, 64, generator=g).to(torch.bfloat16)
    return np.concatenate([_bits(latent), _bits(rope)], axis=1)


def test_every_bf16_value_in_range_rounds_like_the_oracle():
    # one 448 per group sets scale 1, so each code is the e4m3 rounding of the bf16 value itself
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    keep = bits[np.isfinite(vals) & (np.abs(vals) <= 448)]
    per = 127
    n_groups = (keep.size + per - 1) // per
    n_rows = (n_groups + 3) // 4
    latent = np.zeros((n_rows * 4, 128), dtype=np.uint16)
    latent[:, 0] = 0x43E0                                  # 448.0
    flat = np.zeros(n_rows * 4 * per, dtype=np.uint16)
    flat[:keep.size] = keep
    latent[:, 1:] = flat.reshape(n_rows * 4, per)
    src = np.concatenate([latent.reshape(n_rows, 512), np.full((n_rows, 64), 0x3F80, dtype=np.uint16)], axis=1)
    say(f"quantize: every in-range bf16 value, {n_rows} rows")
    cache = np.zeros((((n_rows + 63) // 64) * 64, 656), dtype=np.uint8)
    slots = np.arange(n_rows)
    got = _gpu_write(src, slots, cache)
    want = append_rows(cache, slots, src)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("n,seed", [(1, 0), (7, 1), (3000, 2)])
def test_random_rows_bit_exact(n, seed):
    say(f"quantize: random rows n={n} seed={seed}")
    src = _random_rows(max(n, 7), seed)[-n:]
    num_rows = ((n + 63) // 64 + 1) * 64
    rng = np.random.default_rng(seed)
    cache = rng.integers(0, 256, (num_rows, 656), dtype=np.uint8)
    slots = rng.permutation(num_rows)[:n]
    got = _gpu_write(src, slots, cache)
    assert np.array_equal(got, append_rows(cache, slots, src))


def test_slots_outside_the_cache_write_nothing():
    say("quantize: invalid slots")
    n, num_rows = 200, 4 * 64
    src = _random_rows(n, 3)
    rng = np.random.default_rng(3)
    cache = rng.integers(0, 256, (num_rows, 656), dtype=np.uint8)
    slots = rng.permutation(num_rows)[:n].astype(np.int64)
    slots[::7] = -1
    slots[3] = num_rows
    slots[10] = np.iinfo(np.int32).max
    slots[11] = np.iinfo(np.int32).min
    got = _gpu_write(src, slots, cache)
    assert np.array_equal(got, append_rows(cache, slots, src))


def test_empty_call_is_a_no_op():
    say("quantize: n = 0")
    kv = torch.full((2, 64, 656), 7, dtype=torch.uint8, device=DEV)
    mla.quantize_fp8_append(torch.empty((0, 576), dtype=torch.bfloat16, device=DEV),
                            torch.empty((0,), dtype=torch.int32, device=DEV), kv)
    torch.cuda.synchronize()
    assert bool((kv == 7).all())


def test_full_cache_of_the_fp8_causal_workload_sampled():
    # 64 sequences x 8192 tokens = 524,288 rows into 8192 shuffled pages (the FP8 causal decode's cache)
    B, L = 64, 8192
    n = B * L
    say(f"quantize: full cache n={n}")
    g = torch.Generator().manual_seed(4)
    src = torch.randn(n, 576, generator=g).to(torch.bfloat16)
    pages = torch.randperm(n // 64, generator=g).to(torch.int32)
    t = torch.arange(n, dtype=torch.int32)
    slots = pages[t // 64] * 64 + t % 64
    kv = torch.zeros((n // 64, 64, 656), dtype=torch.uint8, device=DEV)
    mla.quantize_fp8_append(src.to(DEV), slots.to(DEV), kv)
    torch.cuda.synchronize()
    got = kv.view(n, 656)
    pick = torch.randint(0, n, (2048,), generator=g)
    pick[:2] = torch.tensor([0, n - 1])
    want = quantize_rows(_bits(src[pick]))
    assert np.array_equal(got[slots[pick].long().to(DEV)].cpu().numpy(), want)
    # every row was written: no row keeps the zero fill (a written row's scales are never 0)
    assert bool((got[:, 512:528].view(torch.float32) > 0).all())


def test_written_cache_decodes_like_the_oracle():
    # write an FP8 paged cache with the GPU writer, then run the FP8 causal decode on it
    B, s_q, h_q = 2, 2, 128
    lens = [300, 77]
    say("quantize then decode")
    g = torch.Generator().manual_seed(6)
    mbps = max((L + 63) // 64 for L in lens)
    n_blocks = sum((L + 63) // 64 for L in lens) + 1
    perm = torch.randperm(n_blocks, generator=g).to(torch.int32)
    block_table = torch.full((B, mbps), -1, dtype=torch.int32)
    src_rows, slots, p = [], [], 0
    for b, L in enumerate(lens):
        nb = (L + 63) // 64
        block_table[b, :nb] = perm[p:p + nb]
        p += nb
        t = torch.arange(L, dtype=torch.int32)
        slots.append(block_table[b, t // 64] * 64 + t % 64)
        src_rows.append(torch.randn(L, 576, generator=g).to(torch.bfloat16))
    src = torch.cat(src_rows)
    slots = torch.cat(slots)
    kv = torch.zeros((n_blocks, 64, 656), dtype=torch.uint8, device=DEV)
    mla.quantize_fp8_append(src.to(DEV), slots.to(DEV), kv)
    q = torch.randn(B, s_q, h_q, 576, generator=g).to(torch.bfloat16)
    seqlens = torch.tensor(lens, dtype=torch.int32)
    scale = float(np.float32(576 ** -0.5))
    tm, so = mla.get_mla_metadata(seqlens.to(DEV), s_q, h_q)
    o, lse = mla.mla_decode_with_kvcache(q.to(DEV), kv, block_table.to(DEV), seqlens.to(DEV), 512, tm, so,
                                         softmax_scale=scale, causal=True, is_fp8_kvcache=True)
    torch.cuda.synchronize()
    cache = np.zeros((n_blocks * 64, 656), dtype=np.uint8)
    cache = append_rows(cache, slots.numpy(), _bits(src))
    assert np.array_equal(kv.view(-1, 656).cpu().numpy(), cache)
    o_ref, lse_ref = mla_decode_ref(_bits(q), cache.reshape(n_blocks, 64, 656), "fp8", block_table=block_table.numpy(),
                                    cache_seqlens=seqlens.numpy(), softmax_scale=scale, causal=True)
    w = Workload("quantize then decode", q, torch.from_numpy(cache.reshape(n_blocks, 64, 656)), "fp8", block_table,
                 seqlens, None, scale, True)
    compare(o, lse, o_ref, lse_ref, label="quantize then decode", floor_fn=workload_floor_fn(w))
