"""Reference split-KV work schedule (the metadata step), in plain Python loops.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Role, from "矩阵、注意力与 GPU：拆解 DeepGEMM 与 FlashMLA" (msy.plus) §七
"split-KV：把长序列切开": a metadata call, made once per decode step and
reused by every layer, states which sequences, which KV blocks and how many
splits each processor part takes. The pages give no format or balancing rule,
so this is the library's own documented rule, written here as a per-tile
assignment (the GPU computes the same result per part, in parallel):

  * The query rows of sequence b are its rows of q in order, (position i,
    head h) -> i * h_q + h. A dense call puts all s_q * h_q of them in one
    row space, since every position reads the same cache ([Walkthrough] §七
    "先算清楚瓶颈" counts a request's h_q * s_q query rows against one pass
    over the KV); a sparse call has one row space of h_q rows per position, each with
    its own indices. Work units are "row-group sequences" q = b * n_rg + rg,
    rg = i * n_hb + hb (row space i, block hb of rg_rows consecutive rows).
    Unit q has T_q tiles of 64 tokens: ceil(L_b / 64) dense, ceil(topk / 64)
    sparse, with L_b read as at most 2^23 (the longest sequence a call
    attends).
  * Units are laid end to end on a line; a non-empty unit first takes
    fixed_cost positions (its per-split overhead), then one position per tile.
  * With total = sum over non-empty units of (fixed_cost + T_q) and
    W = max(ceil(total / num_parts), min_payload), the tile at position x
    belongs to part floor(x / W).
  * A unit's splits are the distinct parts among its tiles, in order.
  * Placement on the grid: with used = ceil(total / W) work parts that can
    hold tiles and num_parts a multiple of 8, work part j is written to row
    (j // k) * (num_parts // 8) + j % k of tile_meta, k = ceil(used / 8);
    every other row is empty. (The decode grid runs row r on XCD
    r // (num_parts // 8), so the parts holding work are spread over all
    eight XCDs, k consecutive ones each.) Otherwise work part j is row j.
"""

from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 64
MAX_SEQ_TOKENS = 1 << 23


def tile_counts(cache_seqlens: Optional[Sequence[int]], batch: int, s_q: int, h_q: int,
                topk: int, rg_rows: int) -> List[int]:
    """T_q for every row-group sequence, in q order."""
    rows = h_q if topk > 0 else s_q * h_q   # rows of one row space
    n_pos = s_q if topk > 0 else 1           # row spaces per sequence
    n_hb = -(-rows // rg_rows)
    n_rg = n_pos * n_hb
    out = []
    for b in range(batch):
        L = min(max(int(cache_seqlens[b]), 0), MAX_SEQ_TOKENS)
        T = -(-topk // BLOCK_SIZE) if topk > 0 else -(-L // BLOCK_SIZE)
        out.extend([T] * n_rg)
    return out


def split_schedule(T: Sequence[int], num_parts: int, fixed_cost: int, min_payload: int
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Returns (tile_meta int32 [num_parts, 8], split_offsets int32 [Q + 1]).

    tile_meta[p] = [q_begin, t_begin, q_end, t_end (inclusive), first_split,
                    empty (1/0), 0, 0]; an empty part has all zeros but the
    empty flag. split_offsets is the prefix sum of per-unit split counts.
    """
    total = sum(fixed_cost + t for t in T if t > 0)
    W = max(-(-total // num_parts) if total > 0 else 1, min_payload, 1)
    owner: Dict[Tuple[int, int], int] = {}
    pos = 0
    for q, t_count in enumerate(T):
        if t_count <= 0:
            continue
        pos += fixed_cost
        for t in range(t_count):
            owner[(q, t)] = pos // W
            pos += 1
    parts: List[List[Tuple[int, int]]] = [[] for _ in range(num_parts)]
    for (q, t), p in owner.items():  # dict keeps insertion (q, t) order
        assert p < num_parts
        parts[p].append((q, t))
    n_splits = [0] * len(T)
    for q, t_count in enumerate(T):
        if t_count > 0:
            n_splits[q] = len({owner[(q, t)] for t in range(t_count)})
    split_offsets = np.zeros(len(T) + 1, dtype=np.int32)
    split_offsets[1:] = np.cumsum(n_splits)
    used = -(-total // W) if total > 0 else 0
    row_of = list(range(num_parts))
    if num_parts % 8 == 0:
        per_xcd = num_parts // 8
        k = -(-used // 8)
        row_of = [None] * num_parts
        for j in range(used):
            row_of[j] = (j // k) * per_xcd + j % k
    meta = np.zeros((num_parts, 8), dtype=np.int32)
    meta[:, 5] = 1
    for p, tiles in enumerate(parts):
        if not tiles:
            continue
        qb, tb = tiles[0]
        qe, te = tiles[-1]
        first_split = len({owner[(qb, t)] for t in range(tb)})
        meta[row_of[p], :6] = [qb, tb, qe, te, first_split, 0]
    return meta, split_offsets
