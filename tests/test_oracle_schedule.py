"""Pins for the reference split schedule (CPU only): hand-worked cases and invariants."""

import json
import os

import numpy as np
import pytest

from oracle import split_schedule, tile_counts

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_cases():
    with open(os.path.join(GOLDEN, "schedule_small.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        meta, offs = split_schedule(c["T"], c["num_parts"], c["fixed_cost"], c["min_payload"])
        assert meta.tolist() == c["tile_meta"], c["worked"]
        assert offs.tolist() == c["split_offsets"], c["worked"]


def _expand(meta, T):
    """All (q, t) tiles of each part, walking q in order from its begin to its end."""
    out = []
    for row in meta:
        qb, tb, qe, te, fs, empty = row[:6]
        tiles = []
        if not empty:
            for q in range(qb, qe + 1):
                t0 = tb if q == qb else 0
                t1 = te if q == qe else T[q] - 1
                tiles += [(q, t) for t in range(t0, t1 + 1)]
        out.append(tiles)
    return out


@pytest.mark.parametrize("seed", range(20))
def test_invariants_random(seed):
    rng = np.random.default_rng(seed)
    Q = int(rng.integers(1, 40))
    T = [int(x) for x in rng.integers(0, 50, Q)]
    if seed % 5 == 0:
        T[int(rng.integers(0, Q))] = 0
    P = int(rng.choice([1, 3, 8, 64, 256]))
    C = int(rng.integers(0, 5))
    Wmin = int(rng.integers(1, 8))
    meta, offs = split_schedule(T, P, C, Wmin)
    parts = _expand(meta, T)
    seen = [t for p in parts for t in p]
    # every tile exactly once, in (q, t) order across parts
    assert seen == [(q, t) for q in range(Q) for t in range(T[q])]
    # split counts and first_split agree with the parts
    n_splits = np.diff(offs)
    for q in range(Q):
        owners = [p for p, tiles in enumerate(parts) if any(x[0] == q for x in tiles)]
        assert n_splits[q] == len(owners)
        for k, p in enumerate(owners):
            if parts[p][0][0] == q:
                assert meta[p][4] == k
    # balance: no part holds more than W positions (tiles plus overheads it starts)
    total = sum(C + t for t in T if t > 0)
    W = max(-(-total // P) if total else 1, Wmin)
    for tiles in parts:
        assert len(tiles) <= W


def test_tile_counts_layout():
    # h_q = 128 with 128-row groups, s_q = 2: two row groups per batch entry
    assert tile_counts([64, 65, 0], 3, 2, 128, 0, 128) == [1, 1, 2, 2, 0, 0]
    # 20 rows cut into 16-row groups: two row blocks (rows 0-15 and 16-19)
    assert tile_counts([130], 1, 1, 20, 0, 16) == [3, 3]
    # sparse ignores cache_seqlens
    assert tile_counts([5, 5], 2, 1, 128, 2048, 128) == [32, 32]
    # dense calls pack the s_q positions of a sequence into one row space
    # (s_q * h_q rows), sparse calls keep one row space per position
    assert tile_counts([100, 200], 2, 2, 16, 0, 64) == [2, 4]
    assert tile_counts([100, 200], 2, 2, 16, 2048, 16) == [32] * 4
    assert tile_counts([130], 1, 4, 40, 0, 128) == [3, 3]


@pytest.mark.parametrize("seed", range(10))
def test_placement_spreads_work_over_xcds(seed):
    # num_parts a multiple of 8: the rows holding work lie in the first k rows
    # of each of the eight row blocks (one block per XCD); a work part that
    # holds only fixed-cost positions, or lies past the last tile, is empty
    rng = np.random.default_rng(100 + seed)
    Q = int(rng.integers(1, 30))
    T = [int(x) for x in rng.integers(0, 40, Q)]
    P = int(rng.choice([8, 16, 64, 256]))
    C, Wmin = int(rng.integers(0, 4)), int(rng.integers(1, 9))
    meta, _ = split_schedule(T, P, C, Wmin)
    total = sum(C + t for t in T if t > 0)
    W = max(-(-total // P) if total else 1, Wmin)
    used = -(-total // W) if total else 0
    k = -(-used // 8)
    per = P // 8
    busy = meta[:, 5] == 0
    for x in range(8):
        blk = busy[x * per:(x + 1) * per]
        assert not blk[k:].any()
    assert int(busy.sum()) <= used


def test_coverage_checker_catches_planted_schedules():
    """The GPU-side coverage checker (tests/test_gpu_metadata.py) rejects
    schedules with a missing tile, a tile taken twice, a wrong split count
    and a wrong split index, and accepts the reference schedule."""
    import importlib.util
    import os

    spec = importlib.util.spec_from_file_location(
        "gpu_meta", os.path.join(os.path.dirname(__file__), "test_gpu_metadata.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    check = mod.check_covers_every_tile_once
    T = [5, 0, 3, 9, 1]
    meta, off = split_schedule(T, 8, 2, 3)
    check(meta, off, T)
    live = [r for r in range(8) if meta[r, 5] == 0]
    bad = meta.copy()
    bad[live[0], 3] -= 1                     # a tile nobody takes
    bad2 = meta.copy()
    bad2[live[1], 1] = max(0, bad2[live[1], 1] - 1)   # a tile taken twice (or a gap elsewhere)
    bad3 = off.copy()
    bad3[1:] += 1                            # split counts off by one
    bad4 = meta.copy()
    bad4[live[1], 4] += 1                    # wrong first split index
    for m, o in ((bad, off), (bad2, off), (meta, bad3), (bad4, off)):
        with pytest.raises(AssertionError):
            check(m, o, T)


def test_lengths_past_the_longest_sequence_read_as_it():
    """cache_seqlens entries above 2^23 tokens count 2^17 tiles (the
    documented bound that keeps every schedule position below 2^31)."""
    assert tile_counts([(1 << 23) + 5, (1 << 31) - 1, 1 << 23], 3, 1, 16, 0, 16) == [1 << 17] * 3
