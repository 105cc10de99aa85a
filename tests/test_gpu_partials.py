"""Split partials travel as fp16 rows with a power-of-two scale per (split, row).

A sequence split many ways (one fp16 partial per split, merged by the combine)
must give the same o as the same sequence in one split (finished by the split
kernel, no partial) up to the bf16 rounding of o itself, and cache values far
outside fp16's range must not overflow the partial rows.
"""

import numpy as np
import pytest
import torch

from workload import make_workload

from tests.gpu_helpers import compare, oracle, run_gpu, say, workload_floor_fn

pytestmark = pytest.mark.gpu

# Two bf16 results of the same rows, each within half a bf16 ulp of its own
# fp32 value: they differ by at most one ulp at the row's largest |o|
# (2^-7 of it); the fp16 partials add about 2^-12 of each partial row's size.
ROW_REL = 2.0 ** -6


def _row_diff(o_a, o_b):
    a = o_a.float().cpu().numpy().astype(np.float64)
    b = o_b.float().cpu().numpy().astype(np.float64)
    m = np.max(np.abs(b), axis=-1, keepdims=True)
    return float(np.max(np.abs(a - b) / np.maximum(m, 1e-30)))


@pytest.mark.parametrize("fmt,h_q,causal", [("bf16", 128, False), ("bf16", 16, False), ("bf16", 64, False),
                                            ("fp8", 128, True)])
def test_many_splits_match_one_split(fmt, h_q, causal):
    say(f"partials: {fmt} h_q={h_q} causal={causal}, one part against 256")
    s_q = 2 if causal else 1
    w = make_workload(batch=2, s_q=s_q, h_q=h_q, seqlens=[4096, 2999], kv_format=fmt, causal=causal, seed=21)
    o1, l1, _, so1 = run_gpu(w, num_parts=1)
    om, lm, _, som = run_gpu(w, num_parts=256)
    torch.cuda.synchronize()
    n1 = np.diff(so1.cpu().numpy())
    nm = np.diff(som.cpu().numpy())
    assert np.all(n1 == 1) and np.min(nm) >= 8, (n1, nm)   # one split each against many
    d = _row_diff(om, o1)
    dl = float(torch.max(torch.abs(lm - l1)).item())
    say(f"  max |o_many - o_one| / row max = {d:.3e} (bound {ROW_REL:.3e}); max |dlse| = {dl:.3e}")
    assert d <= ROW_REL
    assert dl <= 1e-4


def test_large_magnitude_cache_does_not_overflow_fp16_partials():
    """Latent values up to ~1.6e6 (fp16's largest finite value is 65504) with
    the query scaled down so the scores stay moderate: the merged o matches the
    oracle relative to each row's size, and equals the one-split result."""
    say("partials: bf16 cache scaled by 3e5, q by 1e-5")
    w = make_workload(batch=2, s_q=1, h_q=128, seqlens=[3000, 1500], kv_format="bf16", seed=22)
    kv = w.kv.view(torch.bfloat16)
    w.kv = (kv.float() * 3e5).to(torch.bfloat16).view(torch.uint8)
    w.q = (w.q.float() * 1e-5).to(torch.bfloat16)
    assert float(w.kv.view(torch.bfloat16).float().abs().max()) > 65504 * 4
    om, lm, _, som = run_gpu(w, num_parts=256)
    o1, l1, _, _ = run_gpu(w, num_parts=1)
    torch.cuda.synchronize()
    assert np.min(np.diff(som.cpu().numpy())) >= 8
    assert torch.isfinite(om.float()).all() and torch.isfinite(lm).all()
    d = _row_diff(om, o1)
    say(f"  max |o_many - o_one| / row max = {d:.3e}")
    assert d <= ROW_REL
    o_ref, lse_ref = oracle(w)
    og = om.float().cpu().numpy().astype(np.float64)
    m = np.max(np.abs(o_ref), axis=-1, keepdims=True)
    rel = float(np.max(np.abs(og - o_ref) / m))
    say(f"  max |o - o_ref| / row max = {rel:.3e}")
    assert rel <= ROW_REL
    # lse is unaffected by the value scale: the usual tolerance
    compare(torch.zeros_like(om), lm, np.zeros_like(o_ref), lse_ref, label="lse of the scaled cache",
            floor_fn=workload_floor_fn(w))
