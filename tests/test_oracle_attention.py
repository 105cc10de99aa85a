"""Pins for the oracle's attention, masking, paging and split merge (CPU only).

Each check compares the oracle against something fixed outside it: a library
attention routine, a closed form, an invariant the pages state, or a
hand-derivable special case.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attend, attended_rows, lse_merge, mla_decode_ref

SCALE = float(np.float32(576 ** -0.5))


def _paged(rng, lens, num_extra=3, d=576):
    """fp64 rows laid out in shuffled 64-token pages; returns (rows, block_table)."""
    pages = [-(-l // 64) for l in lens]
    pool = sum(pages) + num_extra
    rows = rng.standard_normal((pool * 64, d))
    perm = rng.permutation(pool)
    bt = np.full((len(lens), max(pages + [1])), -1, dtype=np.int64)
    off = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[off:off + n]
        off += n
    return rows, bt


def _run(q, rows, bt, lens, causal=False, indices=None, scale=SCALE):
    return mla_decode_ref(q, rows, "bf16", block_table=bt, cache_seqlens=np.asarray(lens),
                          softmax_scale=scale, causal=causal, indices=indices, kv_is_decoded=True)


def test_absorbed_equals_unabsorbed_mha():
    """(a) Explicit per-head up-projections W_UK, W_UV with library attention
    (torch SDPA, float64) equal the absorbed MQA form run through the oracle:
    q~ = W_UK^T q^C scores the latent directly and W_UV maps the latent output
    back (walkthrough §六 "吸收")."""
    rng = np.random.default_rng(1)
    h, dh, dc, dr, L = 4, 128, 512, 64, 150
    lens = [L]
    rows, bt = _paged(rng, lens)
    W_UK = rng.standard_normal((h, dh, dc)) / math.sqrt(dc)
    W_UV = rng.standard_normal((h, dh, dc)) / math.sqrt(dc)
    qC = rng.standard_normal((h, dh))
    qR = rng.standard_normal((h, dr))
    q_abs = np.concatenate([np.einsum("hdc,hd->hc", W_UK, qC), qR], axis=1)
    o_lat, lse = _run(q_abs[None, None], rows, bt, lens)
    # explicit keys/values for the L cached tokens, in sequence order
    t = np.arange(L)
    tok = rows[bt[0, t // 64] * 64 + t % 64]
    c, kR = tok[:, :512], tok[:, 512:]
    for hh in range(h):
        k = np.concatenate([c @ W_UK[hh].T, kR], axis=1)      # [L, 192]
        v = c @ W_UV[hh].T                                   # [L, 128]
        qf = np.concatenate([qC[hh], qR[hh]])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qf)[None, None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
            scale=SCALE)[0, 0].numpy()
        assert np.max(np.abs(W_UV[hh] @ o_lat[0, 0, hh] - ref)) < 1e-10
        s = torch.from_numpy(k) @ torch.from_numpy(qf) * SCALE
        assert abs(lse[0, 0, hh] - torch.logsumexp(s, 0).item()) < 1e-10


def test_single_token_returns_its_latent():
    """(b) With one cached token, o is that token's latent; lse is its score."""
    rng = np.random.default_rng(2)
    rows, bt = _paged(rng, [1])
    q = rng.standard_normal((1, 1, 8, 576))
    o, lse = _run(q, rows, bt, [1])
    r = bt[0, 0] * 64
    assert np.array_equal(o[0, 0], np.broadcast_to(rows[r, :512], (8, 512)))
    assert np.allclose(lse[0, 0], SCALE * (q[0, 0] @ rows[r]), rtol=0, atol=1e-13)


def test_equal_scores_give_mean_of_latents():
    """(c) When every key scores the same (zero latent query, identical rope
    keys), o is the plain mean of the latents and lse = ln n + score."""
    rng = np.random.default_rng(3)
    L = 200
    rows, bt = _paged(rng, [L])
    rows[:, 512:] = rng.standard_normal(64)  # identical rope part everywhere
    q = np.zeros((1, 1, 3, 576))
    q[..., 512:] = rng.standard_normal((3, 64))
    o, lse = _run(q, rows, bt, [L])
    t = np.arange(L)
    lat = rows[bt[0, t // 64] * 64 + t % 64, :512]
    s0 = SCALE * (q[0, 0, :, 512:] @ rows[0, 512:])
    assert np.max(np.abs(o[0, 0] - lat.mean(axis=0))) < 1e-12
    assert np.max(np.abs(lse[0, 0] - (math.log(L) + s0))) < 1e-12


def test_sparse_all_rows_equals_dense_and_ignores_invalid():
    """(d) Sparse attention over every row of the sequence, in order, equals
    dense bit for bit; -1 entries (and out-of-range rows) change nothing."""
    rng = np.random.default_rng(4)
    lens = [130, 64]
    rows, bt = _paged(rng, lens)
    q = rng.standard_normal((2, 1, 5, 576))
    od, ld = _run(q, rows, bt, lens)
    for b, L in enumerate(lens):
        t = np.arange(L)
        full = bt[b, t // 64] * 64 + t % 64
        idx = np.full((2, 1, L + 7), -1, dtype=np.int64)
        idx[b, 0, :L] = full
        os_, ls = _run(q, rows, None, lens, indices=idx)
        assert np.array_equal(os_[b], od[b]) and np.array_equal(ls[b], ld[b])
        # scatter -1 and out-of-range values between the real entries
        pos = np.sort(rng.choice(L + 7, L, replace=False))
        idx2 = np.full((2, 1, L + 7), -1, dtype=np.int64)
        idx2[b, 0, pos] = full
        holes = np.setdiff1d(np.arange(L + 7), pos)
        idx2[b, 0, holes[:3]] = rows.shape[0] + np.arange(3)
        os2, ls2 = _run(q, rows, None, lens, indices=idx2)
        assert np.array_equal(os2[b], od[b]) and np.array_equal(ls2[b], ld[b])


def test_split_merge_identity():
    """(e) Merging the oracle's results on two disjoint key sets with the split
    merge equals the oracle on their union (walkthrough §七 split-KV)."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((6, 576))
    K = rng.standard_normal((300, 576)) * 2.0
    o_all, l_all = attend(q, K, SCALE)
    for cut in (1, 57, 299):
        o1, l1 = attend(q, K[:cut], SCALE)
        o2, l2 = attend(q, K[cut:], SCALE)
        o, l = lse_merge(np.stack([o1, o2]), np.stack([l1, l2]))
        assert np.max(np.abs(o - o_all)) < 1e-12 and np.max(np.abs(l - l_all)) < 1e-12
    # an empty part weighs nothing; all-empty gives o = 0, lse = -inf
    oe, le = attend(q, K[:0], SCALE)
    o, l = lse_merge(np.stack([o_all, oe]), np.stack([l_all, le]))
    assert np.array_equal(o, o_all) and np.array_equal(l, l_all)
    o, l = lse_merge(np.stack([oe, oe]), np.stack([le, le]))
    assert np.all(o == 0) and np.all(l == -np.inf)


def test_causal_alignment():
    """(f) Bottom-right causal: the last query row equals non-causal; query i
    equals dense attention over the first L - s_q + 1 + i tokens."""
    rng = np.random.default_rng(6)
    L, s_q = 150, 3
    rows, bt = _paged(rng, [L])
    q = rng.standard_normal((1, s_q, 4, 576))
    oc, lc = _run(q, rows, bt, [L], causal=True)
    on, ln = _run(q, rows, bt, [L], causal=False)
    assert np.array_equal(oc[0, s_q - 1], on[0, s_q - 1])
    for i in range(s_q):
        Li = L - s_q + 1 + i
        oi, li = _run(q[:, i:i + 1], rows, bt, [Li])
        assert np.array_equal(oc[0, i], oi[0, 0]) and np.array_equal(lc[0, i], li[0, 0])
    assert not np.array_equal(oc[0, 0], on[0, 0])


def test_page_permutation_invariance():
    """(g) Moving pages in the pool and remapping block_table changes nothing."""
    rng = np.random.default_rng(7)
    lens = [100, 257]
    rows, bt = _paged(rng, lens)
    q = rng.standard_normal((2, 1, 4, 576))
    o, l = _run(q, rows, bt, lens)
    pool = rows.shape[0] // 64
    perm = rng.permutation(pool)             # page p moves to slot perm[p]
    rows2 = np.empty_like(rows)
    for p in range(pool):
        rows2[perm[p] * 64:(perm[p] + 1) * 64] = rows[p * 64:(p + 1) * 64]
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1)
    o2, l2 = _run(q, rows2, bt2, lens)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


@pytest.mark.parametrize("n", [2, 3])
def test_brute_force_small_against_scipy(n):
    """(j) One head, n keys: library softmax / logsumexp on the same scores."""
    rng = np.random.default_rng(10 + n)
    q = rng.standard_normal((1, 576))
    K = rng.standard_normal((n, 576))
    o, lse = attend(q, K, SCALE)
    s = np.array([SCALE * float(np.dot(q[0], K[j])) for j in range(n)])
    p = scipy.special.softmax(s)
    assert np.max(np.abs(o[0] - p @ K[:, :512])) < 1e-14
    assert abs(lse[0] - scipy.special.logsumexp(s)) < 1e-14


def test_empty_sets():
    rng = np.random.default_rng(8)
    rows, bt = _paged(rng, [5, 0])
    q = rng.standard_normal((2, 1, 3, 576))
    o, l = _run(q, rows, bt, [5, 0])
    assert np.all(o[1] == 0) and np.all(l[1] == -np.inf)
    idx = np.full((2, 1, 4), -1)
    o, l = _run(q, rows, None, [5, 0], indices=idx)
    assert np.all(o == 0) and np.all(l == -np.inf)


def test_invalid_pages_and_positions_past_the_table_are_skipped():
    """Dense positions whose page id names no cache page (-1, or a page past
    the pool) and positions past the block table's row contribute nothing:
    o and lse equal library softmax / logsumexp over the scores of the
    remaining tokens, gathered by hand."""
    rng = np.random.default_rng(12)
    rows, bt = _paged(rng, [300], num_extra=2)   # 5 pages of 64 in a pool of 7
    pool = rows.shape[0] // 64
    q = rng.standard_normal((1, 1, 3, 576))

    def check(table, L, kept_positions):
        o, lse = _run(q, rows, table, [L])
        K = rows[[int(bt[0, t // 64]) * 64 + t % 64 for t in kept_positions]]
        for h in range(3):
            s = SCALE * (K @ q[0, 0, h])
            assert np.max(np.abs(o[0, 0, h] - scipy.special.softmax(s) @ K[:, :512])) < 1e-12
            assert abs(lse[0, 0, h] - scipy.special.logsumexp(s)) < 1e-12

    bad = bt.copy()
    bad[0, 1] = -1          # positions 64..127
    bad[0, 3] = pool + 2    # positions 192..255: a page id past the cache
    check(bad, 300, [t for t in range(300) if t // 64 in (0, 2, 4)])
    # a block table of two pages holds positions 0..127 only, whatever L says
    check(np.ascontiguousarray(bt[:, :2]), 200, list(range(128)))


def test_attended_rows_dense_mapping():
    bt = np.array([[3, 0, 7]])
    r = attended_rows(0, 0, s_q=1, num_rows=8 * 64, block_table=bt, cache_seqlens=np.array([130]),
                      causal=False, indices=None)
    assert list(r[:2]) == [192, 193] and r[64] == 0 and r[128] == 7 * 64 and r[129] == 7 * 64 + 1
    assert len(r) == 130


def test_sparse_with_causal_rejected():
    rng = np.random.default_rng(9)
    rows, bt = _paged(rng, [5])
    with pytest.raises(ValueError):
        _run(rng.standard_normal((1, 1, 2, 576)), rows, bt, [5], causal=True, indices=np.zeros((1, 1, 1), int))
