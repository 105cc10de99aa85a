"""The largest shapes the library takes.

One call holds at most 8192 row-group sequences and 65535 parts, and the
schedule reads a sequence as at most 2^23 tokens (2^17 tiles). At those sizes
the split schedule equals the oracle's bit for bit and covers every tile once,
and the decode with 8192 row-group sequences matches the oracle ([Walkthrough]
§七: every KV block of every sequence is processed by exactly one split)."""

import dataclasses

import numpy as np
import pytest
import torch

import mla_latent_kv_10_amd as mla
from oracle import split_schedule, tile_counts
from workload import make_workload

from tests.gpu_helpers import compare, oracle, run_gpu, say, workload_floor_fn
from tests.test_gpu_metadata import _policy, check_covers_every_tile_once

pytestmark = pytest.mark.gpu

MAX_UNITS = 8192
MAX_PARTS = 65535
LONGEST = 1 << 23


def _lens(n, hi, seed):
    g = np.random.default_rng(seed)
    lens = g.integers(0, hi + 1, n)
    lens[g.random(n) < 0.1] = 0
    return lens


# (label, lengths, s_q, h_q, num_parts, topk)
SCHEDULE_CASES = [
    ("8192 16-row sequences, 65535 parts", _lens(8192, 6400, 1), 1, 16, MAX_PARTS, 0),
    ("8192 16-row sequences, 65528 parts (spread over the XCDs)", _lens(8192, 6400, 2), 1, 16, 65528, 0),
    ("4096 batches of two 128-row groups, 1024 parts", _lens(4096, 6400, 3), 2, 128, 1024, 0),
    ("8192 64-row sequences, 256 parts", _lens(8192, 3000, 4), 1, 64, 256, 0),
    ("longest sequences, 256 parts", np.array([LONGEST, LONGEST - 1, LONGEST + 100, 0]), 1, 16, 256, 0),
    ("longest sequences, one part", np.array([LONGEST, 1, LONGEST + 100]), 1, 128, 1, 0),
    ("sparse, topk 2^23", np.zeros(2, dtype=np.int64), 1, 128, 256, LONGEST),
    ("sparse, 8192 sequences", np.zeros(8192, dtype=np.int64), 1, 16, 4096, 2048),
]


@pytest.mark.parametrize("label,lens,s_q,h_q,num_parts,topk", SCHEDULE_CASES, ids=[c[0] for c in SCHEDULE_CASES])
def test_schedule_at_the_largest_shapes(label, lens, s_q, h_q, num_parts, topk):
    batch = len(lens)
    say(f"schedule at the limits: {label}")
    seq = torch.tensor(lens.astype(np.int64), dtype=torch.int32, device="cuda:0")
    tm, so = mla.get_mla_metadata(seq if topk == 0 else None, s_q, h_q, topk=topk, num_parts=num_parts,
                                  batch=batch)
    torch.cuda.synchronize()
    rg, C, Wmin = _policy(h_q, s_q, batch, num_parts, topk)
    T = tile_counts(lens.tolist(), batch, s_q, h_q, topk, rg)
    assert len(T) <= MAX_UNITS
    ref_meta, ref_off = split_schedule(T, num_parts, C, Wmin)
    got_off = so.cpu().numpy()[:len(ref_off)]
    got_meta = tm.cpu().numpy()
    assert np.array_equal(got_off, ref_off)
    assert np.array_equal(got_meta, ref_meta)
    check_covers_every_tile_once(got_meta, got_off, T)


# (label, workload arguments, batches compared: None = all)
DECODE_CASES = [
    ("bf16 dense, 8192 16-row sequences",
     dict(batch=8192, s_q=1, h_q=16, seqlen_range=(0, 100), kv_format="bf16"), None),
    ("fp8 dense, 8192 16-row sequences",
     dict(batch=8192, s_q=1, h_q=16, seqlen_range=(0, 100), kv_format="fp8"), None),
    ("bf16 sparse, 8192 16-row sequences",
     dict(batch=8192, s_q=1, h_q=16, kv_format="bf16", topk=64, sparse_tokens_per_seq=128, invalid_frac=0.1),
     None),
    ("bf16 causal s_q=2 h_q=128, 4096 batches of two 128-row groups",
     dict(batch=4096, s_q=2, h_q=128, seqlen_range=(0, 100), kv_format="bf16", causal=True), 48),
]


@pytest.mark.parametrize("label,kw,n_batches", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_with_the_most_sequences(label, kw, n_batches):
    """Every query row, or (n_batches set) every row of the first and last
    batches and a seeded sample of the others: a batch's result depends only
    on its own q, length, block-table row or indices and the shared cache, so
    the oracle runs on a workload of just those batches."""
    say(f"decode at the sequence limit: {label}")
    w = make_workload(**kw, seed=41)
    o, lse, _, _ = run_gpu(w)
    torch.cuda.synchronize()
    if n_batches is not None:
        g = np.random.default_rng(7)
        picks = sorted({0, w.batch - 1} | set(int(b) for b in g.integers(0, w.batch, n_batches)))
        sel = torch.tensor(picks)
        w = dataclasses.replace(
            w, q=w.q[sel].contiguous(), cache_seqlens=w.cache_seqlens[sel].contiguous(),
            block_table=None if w.block_table is None else w.block_table[sel].contiguous(),
            indices=None if w.indices is None else w.indices[sel].contiguous())
        o, lse = o[sel.to(o.device)], lse[sel.to(lse.device)]
    o_ref, lse_ref = oracle(w)
    compare(o, lse, o_ref, lse_ref, label=label, floor_fn=workload_floor_fn(w))
