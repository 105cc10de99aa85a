"""LDS race check: the pipelined split kernel against its race-check build.

The race-check build (libmla_mi355x_drain.so, MLA_DRAIN_PIPELINE) waits for
every tile's loads right after issuing them, so the loads of tile k + 1 or
k + 2 land in LDS at the earliest point the schedule allows instead of
somewhere during tile k. The arithmetic is the same instruction for
instruction, so with the same schedule the outputs must be equal bit for bit;
a load issued into a buffer that some wave still reads would make them differ.
Every pipeline is covered: FP8 with 128-row groups (loads between the score
MFMAs, sparse index ring), bf16 with 128- and 64-row groups (loads between the
score MFMAs), and the two-tiles-ahead pipeline of FP8 with 64-row groups and
of 16-row groups, dense (with and without row groups that
span query positions) and sparse, each over segments of many tiles."""

import ctypes

import pytest
import torch

import mla_latent_kv_10_amd as mla
from workload import make_workload

from tests.gpu_helpers import run_gpu, say, to_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # fmt, h_q, s_q, causal, sparse
    ("bf16", 128, 1, False, False),
    ("bf16", 128, 2, True, True),
    ("fp8", 128, 2, True, False),
    ("fp8", 128, 1, False, True),
    ("fp8_528", 128, 1, True, False),
    ("fp8_528", 128, 1, False, True),
    ("bf16", 64, 2, True, False),
    ("bf16", 32, 1, False, False),
    ("bf16", 64, 1, False, True),
    ("fp8", 64, 1, False, True),
    ("fp8_528", 48, 1, False, False),
    ("fp8_528", 32, 1, False, True),
    ("bf16", 16, 1, False, False),
    ("bf16", 8, 2, True, False),
    ("fp8", 16, 3, True, False),
    ("fp8_528", 16, 2, True, True),
]


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu()


@pytest.mark.parametrize("num_parts", [16, 256])
@pytest.mark.parametrize("fmt,h_q,s_q,causal,sparse", CASES)
def test_drained_pipeline_is_bit_identical(fmt, h_q, s_q, causal, sparse, num_parts):
    say(f"race check {fmt} h_q={h_q} s_q={s_q} causal={causal} sparse={sparse} parts={num_parts}")
    if sparse:
        w = make_workload(batch=3, s_q=s_q, h_q=h_q, kv_format=fmt, topk=1000, sparse_tokens_per_seq=4096,
                          invalid_frac=0.05, seed=31)
    else:
        w = make_workload(batch=3, s_q=s_q, h_q=h_q, seqlens=[2900, 70, 1313], kv_format=fmt, causal=causal,
                          seed=31)
    g = to_gpu(w)
    o1, lse1, tm, so = run_gpu(w, g, num_parts=num_parts)
    o2 = torch.full_like(o1, float("nan"))
    lse2 = torch.full_like(lse1, float("nan"))
    ws = torch.empty((mla.workspace_size(w.batch, w.s_q, w.h_q, num_parts),), dtype=torch.uint8,
                     device="cuda:0")
    a = mla.make_args(g["q"], g["kv"], g["block_table"], g["cache_seqlens"], tm, so, w.softmax_scale, w.causal,
                      fmt != "bf16", g["indices"], ws, o2, lse2)
    L = mla.drain_lib()
    status = L.mla_decode_with_kvcache(ctypes.byref(a), torch.cuda.current_stream().cuda_stream)
    assert status == mla.MLA_OK, L.mla_last_error()
    torch.cuda.synchronize()
    assert torch.equal(_bits(o1), _bits(o2))
    assert torch.equal(_bits(lse1), _bits(lse2))
