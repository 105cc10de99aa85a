"""mla_decode_with_kvcache_static (the library's static scratch, no
allocation) against mla_decode_with_kvcache with a caller workspace: the same
kernels with the same schedule, so the outputs must agree bit for bit. Two
calls in a row, the second smaller, show the scratch keeps no state that
matters between calls."""

import ctypes

import pytest
import torch

import mla_latent_kv_10_amd as mla
from workload import config_workload, make_workload

from tests.gpu_helpers import run_gpu, say, to_gpu

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu()


def _static(w, g, tm, so):
    o = torch.full((w.batch, w.s_q, w.h_q, 512), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.full((w.batch, w.s_q, w.h_q), float("nan"), dtype=torch.float32, device="cuda:0")
    no_ws = torch.empty((0,), dtype=torch.uint8, device="cuda:0")
    a = mla.make_args(g["q"], g["kv"], g["block_table"], g["cache_seqlens"], tm, so, w.softmax_scale, w.causal,
                      w.kv_format == "fp8", g["indices"], no_ws, o, lse)
    st = mla.lib().mla_decode_with_kvcache_static(ctypes.byref(a), torch.cuda.current_stream().cuda_stream)
    mla.check(st)
    return o, lse


PAIRS = [
    ("dense bf16 h128 then a smaller fp8 causal call",
     lambda: config_workload(2),
     lambda: make_workload(batch=3, s_q=2, h_q=128, seqlens=[700, 65, 1], kv_format="fp8", causal=True, seed=51)),
    ("fp8 causal B=64 then a smaller 16-head call",
     lambda: config_workload(4),
     lambda: make_workload(batch=4, s_q=1, h_q=16, seqlens=[3000, 1, 640, 0], kv_format="bf16", seed=52)),
    ("sparse fp8 then a smaller sparse bf16 64-head call",
     lambda: config_workload(5),
     lambda: make_workload(batch=2, s_q=1, h_q=64, kv_format="bf16", topk=300, sparse_tokens_per_seq=1024,
                           invalid_frac=0.1, seed=53)),
]


@pytest.mark.parametrize("label,first,second", PAIRS, ids=[p[0] for p in PAIRS])
def test_static_scratch_matches_the_workspace_entry(label, first, second):
    for k, make in enumerate((first, second)):
        w = make()
        say(f"static scratch: {label}, call {k + 1}: {w.name} B={w.batch} s_q={w.s_q} h_q={w.h_q}")
        g = to_gpu(w)
        ref_o, ref_lse, tm, so = run_gpu(w, g)
        o, lse = _static(w, g, tm, so)
        torch.cuda.synchronize()
        assert torch.equal(_bits(o), _bits(ref_o)) and torch.equal(_bits(lse), _bits(ref_lse))
