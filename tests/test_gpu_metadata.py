"""Split schedule on the GPU equals the reference schedule bit for bit."""

import numpy as np
import pytest
import torch

import mla_latent_kv_10_amd as mla
from oracle import split_schedule, tile_counts

from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu

# The documented policy (include/mla.h): a row space holds R = s_q * h_q rows
# (dense) or h_q rows per position (sparse); row groups of 16 rows when
# R <= 16, 64 when 16 < R <= 64, else 128; (fixed_cost, min_payload) = (0, 1)
# for 16, (2, 2) for 64 and (2, 3) for 128, with fixed_cost 0 for sparse calls.


def _policy(h_q, s_q, batch, num_parts, topk):
    R = h_q if topk > 0 else s_q * h_q
    if R <= 16:
        rg, C, Wmin = 16, 0, 1
    else:
        rg, C, Wmin = (64, 2, 2) if R <= 64 else (128, 2, 3)
    return rg, (0 if topk > 0 else C), Wmin


CASES = []
rng = np.random.default_rng(0)
for n in range(40):
    batch = int(rng.choice([1, 2, 5, 16, 33, 64, 200]))
    s_q = int(rng.choice([1, 1, 2, 3]))
    h_q = int(rng.choice([4, 16, 20, 64, 100, 128, 130]))
    num_parts = int(rng.choice([1, 3, 8, 64, 256, 300, 1024]))
    topk = int(rng.choice([0, 0, 0, 64, 100, 2048]))
    CASES.append((batch, s_q, h_q, num_parts, topk, int(rng.integers(0, 1 << 30))))
CASES += [(16, 1, 128, 256, 0, 7), (16, 1, 16, 256, 0, 8), (64, 2, 128, 256, 0, 9), (32, 1, 128, 256, 2048, 10),
          (1, 1, 4, 256, 0, 11)]


@pytest.mark.parametrize("batch,s_q,h_q,num_parts,topk,seed", CASES)
def test_metadata_matches_reference(batch, s_q, h_q, num_parts, topk, seed):
    g = np.random.default_rng(seed)
    lens = g.integers(0, 5000, batch)
    lens[g.random(batch) < 0.1] = 0
    lens[g.random(batch) < 0.1] = 1
    say(f"metadata case batch={batch} s_q={s_q} h_q={h_q} parts={num_parts} topk={topk}")
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    tm, so = mla.get_mla_metadata(seq if topk == 0 else None, s_q, h_q, topk=topk, num_parts=num_parts,
                                  batch=batch)
    torch.cuda.synchronize()
    rg, C, Wmin = _policy(h_q, s_q, batch, num_parts, topk)
    T = tile_counts(lens.tolist(), batch, s_q, h_q, topk, rg)
    ref_meta, ref_off = split_schedule(T, num_parts, C, Wmin)
    # the buffer may be longer (its size covers a sparse call of the shape too):
    # the schedule is its first Q + 1 entries
    assert np.array_equal(so.cpu().numpy()[:len(ref_off)], ref_off)
    assert np.array_equal(tm.cpu().numpy(), ref_meta)


def check_covers_every_tile_once(tm, so, T):
    """Properties any correct split schedule has, whatever its balancing rule
    ([Walkthrough] §七: every KV block of every sequence is processed by
    exactly one split, and the split merge needs each sequence's split count):
    every tile (q, t) with t < T[q] lies in exactly one segment; a sequence's
    segments, in KV order, carry split indices 0, 1, ..., n - 1 with
    n = split_offsets[q + 1] - split_offsets[q]; empty rows are all zero but
    the empty flag."""
    Q = len(T)
    so = np.asarray(so, dtype=np.int64)
    assert so.shape == (Q + 1,) and so[0] == 0 and np.all(np.diff(so) >= 0)
    segs = {q: [] for q in range(Q)}
    for r, row in enumerate(np.asarray(tm)):
        qb, tb, qe, te, fs, empty = (int(x) for x in row[:6])
        if empty:
            assert row.tolist() == [0, 0, 0, 0, 0, 1, 0, 0], (r, row)
            continue
        assert row[6] == 0 and row[7] == 0 and 0 <= qb <= qe < Q, (r, row)
        for q in range(qb, qe + 1):
            if T[q] == 0:
                continue
            t0 = tb if q == qb else 0
            t1 = te if q == qe else T[q] - 1
            assert 0 <= t0 <= t1 < T[q], (r, q, t0, t1, T[q])
            segs[q].append((t0, t1, fs if q == qb else 0))
    for q in range(Q):
        s = sorted(segs[q])
        n = int(so[q + 1] - so[q])
        assert len(s) == n, (q, s, n)
        nxt = 0
        for k, (t0, t1, split) in enumerate(s):
            assert t0 == nxt and split == k, (q, s)
            nxt = t1 + 1
        assert nxt == T[q], (q, s, T[q])


@pytest.mark.parametrize("batch,s_q,h_q,num_parts,topk,seed", CASES)
def test_gpu_schedule_covers_every_tile_once(batch, s_q, h_q, num_parts, topk, seed):
    g = np.random.default_rng(seed + 1)
    lens = g.integers(0, 9000, batch)
    lens[g.random(batch) < 0.15] = 0
    say(f"schedule coverage batch={batch} s_q={s_q} h_q={h_q} parts={num_parts} topk={topk}")
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    tm, so = mla.get_mla_metadata(seq if topk == 0 else None, s_q, h_q, topk=topk, num_parts=num_parts,
                                  batch=batch)
    torch.cuda.synchronize()
    R = h_q if topk > 0 else s_q * h_q
    rg = 16 if R <= 16 else (64 if R <= 64 else 128)
    n_rg = (s_q if topk > 0 else 1) * -(-R // rg)
    per_seq = [-(-topk // 64) if topk > 0 else -(-int(L) // 64) for L in lens]
    T = [per_seq[q // n_rg] for q in range(batch * n_rg)]
    check_covers_every_tile_once(tm.cpu().numpy(), so.cpu().numpy()[:len(T) + 1], T)
