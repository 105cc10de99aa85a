"""Bit-exact properties of the HIP path: paging, gather and the masked-token set.

The same metadata (same shapes) is used on both sides of every comparison,
so the arithmetic order is identical and results must match bit for bit."""

import numpy as np
import pytest
import torch

from workload import make_workload

from tests.gpu_helpers import run_gpu, say, to_gpu

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu()


def _same(a, b):
    return torch.equal(_bits(a[0]), _bits(b[0])) and torch.equal(_bits(a[1]), _bits(b[1]))


@pytest.mark.parametrize("fmt,h_q", [("bf16", 128), ("bf16", 16), ("fp8", 128), ("fp8", 16), ("fp8_528", 128),
                                     ("fp8_528", 16)])
def test_page_shuffle_invariance(fmt, h_q):
    say(f"page shuffle {fmt} h_q={h_q}")
    w = make_workload(batch=3, s_q=1, h_q=h_q, seqlens=[700, 129, 64], kv_format=fmt, extra_blocks=5, seed=21)
    base = run_gpu(w)
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(w.num_blocks, generator=g)  # page p moves to slot perm[p]
    kv2 = torch.empty_like(w.kv)
    kv2[perm] = w.kv
    bt2 = torch.where(w.block_table >= 0, perm[w.block_table.clamp(min=0).long()].to(torch.int32), w.block_table)
    w.kv, w.block_table = kv2, bt2
    moved = run_gpu(w)
    torch.cuda.synchronize()
    assert _same(base, moved)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "fp8_528"])
def test_gather_permutation_invariance(fmt):
    say(f"gather permutation {fmt}")
    w = make_workload(batch=2, s_q=1, h_q=128, kv_format=fmt, topk=300, sparse_tokens_per_seq=1024,
                      invalid_frac=0.05, seed=22)
    base = run_gpu(w)
    g = torch.Generator().manual_seed(6)
    n_rows = w.num_blocks * 64
    perm = torch.randperm(n_rows, generator=g)          # row r moves to perm[r]
    flat = w.kv.reshape(n_rows, -1)
    moved = torch.empty_like(flat)
    moved[perm] = flat
    w.kv = moved.reshape(w.kv.shape)
    idx = w.indices.long()
    w.indices = torch.where(idx >= 0, perm[idx.clamp(min=0)], idx).to(torch.int32)
    moved_out = run_gpu(w)
    torch.cuda.synchronize()
    assert _same(base, moved_out)


def _poison_rows(w, keep_rows, value_bytes):
    flat = w.kv.reshape(-1, w.kv.shape[2])
    mask = torch.ones(flat.shape[0], dtype=torch.bool)
    mask[keep_rows] = False
    flat[mask] = value_bytes
    return flat


def _attended_rows(w):
    rows = set()
    for b in range(w.batch):
        for i in range(w.s_q):
            if w.indices is not None:
                for v in w.indices[b, i].tolist():
                    if 0 <= v < w.num_blocks * 64:
                        rows.add(v)
            else:
                L = int(w.cache_seqlens[b])
                lim = L - w.s_q + 1 + i if w.causal else L
                for t in range(max(0, lim)):
                    rows.add(int(w.block_table[b, t // 64]) * 64 + t % 64)
    return torch.tensor(sorted(rows), dtype=torch.long)


@pytest.mark.parametrize("fmt,h_q,causal,sparse", [("bf16", 128, False, False), ("bf16", 16, True, False),
                                                  ("fp8", 128, True, False), ("fp8", 16, False, False),
                                                  ("fp8", 128, False, True), ("bf16", 16, False, True),
                                                  ("fp8_528", 128, True, False), ("fp8_528", 64, False, True)])
def test_nan_poison_of_masked_rows(fmt, h_q, causal, sparse):
    """Every row no query attends to (page tails, causal-excluded tokens,
    unreferenced pages, rows named only by -1) is overwritten with NaN bytes;
    o and lse must not change by a single bit."""
    say(f"nan poison {fmt} h_q={h_q} causal={causal} sparse={sparse}")
    if sparse:
        w = make_workload(batch=2, s_q=1, h_q=h_q, kv_format=fmt, topk=150, sparse_tokens_per_seq=512,
                          invalid_frac=0.1, seed=23)
    else:
        w = make_workload(batch=3, s_q=2 if causal else 1, h_q=h_q, seqlens=[301, 64, 5], kv_format=fmt,
                          causal=causal, extra_blocks=4, seed=23)
        # block_table padding points at a poisoned page instead of -1
        w.block_table[w.block_table < 0] = w.num_blocks - 1
    keep = _attended_rows(w)
    w.kv = w.kv.clone()
    flat = w.kv.reshape(-1, w.kv.shape[2])
    zero = flat.clone()
    zero_mask = torch.ones(flat.shape[0], dtype=torch.bool)
    zero_mask[keep] = False
    zero[zero_mask] = 0
    w.kv = zero.reshape(w.kv.shape)
    clean = run_gpu(w)
    nan = zero.clone()
    nan[zero_mask] = 0xFF  # 0xFFFF bf16 and 0xFF e4m3 are NaN; fp32 scale 0xFFFFFFFF is NaN
    w.kv = nan.reshape(w.kv.shape)
    poisoned = run_gpu(w)
    torch.cuda.synchronize()
    assert _same(clean, poisoned)
    # conversely, changing an attended boundary token changes the output
    last = keep[-1].item()
    bumped = nan.clone()
    bumped[last, :64] = 0x3C if fmt != "bf16" else 0x40
    w.kv = bumped.reshape(w.kv.shape)
    changed = run_gpu(w)
    torch.cuda.synchronize()
    assert not _same(poisoned, changed)


def test_repeat_determinism():
    say("repeat determinism x100")
    w = make_workload(batch=4, s_q=1, h_q=128, seqlens=[3000, 10, 640, 1200], kv_format="bf16", seed=24)
    g = to_gpu(w)
    first = run_gpu(w, g)
    torch.cuda.synchronize()
    for _ in range(99):
        again = run_gpu(w, g)
        assert _same(first, again)


@pytest.mark.parametrize("fmt,h_q,sparse", [("bf16", 128, False), ("fp8", 16, False), ("fp8", 64, True)])
def test_split_then_combine_equals_one_call(fmt, h_q, sparse):
    """mla_decode_splits followed by mla_combine is the same two kernels as
    mla_decode_with_kvcache: outputs agree bit for bit."""
    import mla_latent_kv_10_amd as mla

    say(f"splits+combine vs one call {fmt} h_q={h_q} sparse={sparse}")
    if sparse:
        w = make_workload(batch=2, s_q=1, h_q=h_q, kv_format=fmt, topk=400, sparse_tokens_per_seq=2048,
                          invalid_frac=0.05, seed=25)
    else:
        w = make_workload(batch=3, s_q=1, h_q=h_q, seqlens=[2000, 1, 900], kv_format=fmt, seed=25)
    g = to_gpu(w)
    o1, lse1, tm, so = run_gpu(w, g, num_parts=16)
    o2 = torch.full_like(o1, float("nan"))
    lse2 = torch.full_like(lse1, float("nan"))
    ws = torch.empty((mla.workspace_size(w.batch, w.s_q, w.h_q, 16),), dtype=torch.uint8, device="cuda:0")
    a = mla.make_args(g["q"], g["kv"], g["block_table"], g["cache_seqlens"], tm, so, w.softmax_scale, w.causal,
                      fmt == "fp8", g["indices"], ws, o2, lse2)
    side = torch.cuda.Stream()  # a non-default stream: its handle is a full 64-bit pointer
    side.wait_stream(torch.cuda.current_stream())
    mla.mla_decode_splits(a, side.cuda_stream)
    mla.mla_combine(a, side.cuda_stream)
    torch.cuda.synchronize()
    assert _same((o1, lse1), (o2, lse2))


def _set_latent(flat, row, fmt):
    """Overwrite the latent part of one cache row with large equal values
    (bf16 20.0, or e4m3 code 0x7E = 448, its group's amax after scaling)."""
    if fmt in ("fp8", "fp8_528"):
        flat[row, :512] = 0x7E
    else:
        flat[row, :1024].view(torch.int16)[:] = 0x41A0


@pytest.mark.parametrize("fmt,h_q,causal", [("bf16", 128, False), ("bf16", 16, True), ("fp8", 128, True),
                                            ("fp8", 64, False), ("bf16", 64, True), ("fp8_528", 128, True),
                                            ("fp8_528", 16, False)])
def test_boundary_tokens(fmt, h_q, causal):
    """For every query row (b, i): changing the last token it attends
    (t = L_b - 1, or t = L_b - s_q + i when causal) changes o[b, i], and
    changing the first token past its limit (a page-tail row, or the token the
    next query position adds) leaves o[b, i] and lse[b, i] the same bit for
    bit. The sequences end mid-page, on a page edge and one past it."""
    say(f"boundary tokens {fmt} h_q={h_q} causal={causal}")
    s_q = 2 if causal else 1
    lens = [130, 128, 65]
    w = make_workload(batch=3, s_q=s_q, h_q=h_q, seqlens=lens, kv_format=fmt, causal=causal, extra_blocks=3,
                      seed=31)
    base_kv = w.kv.clone()
    base = run_gpu(w)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        for i in range(s_q):
            last = L - s_q + i if causal else L - 1
            for t, expect_change in ((last, True), (last + 1, False)):
                page = int(w.block_table[b, t // 64]) if t // 64 < w.block_table.shape[1] else -1
                if page < 0:
                    continue  # no cache row holds position t (the sequence ends on a page edge)
                kv = base_kv.clone()
                _set_latent(kv.reshape(-1, kv.shape[2]), page * 64 + t % 64, fmt)
                w.kv = kv
                out = run_gpu(w)
                torch.cuda.synchronize()
                same = (torch.equal(_bits(out[0][b, i]), _bits(base[0][b, i]))
                        and torch.equal(_bits(out[1][b, i]), _bits(base[1][b, i])))
                assert same != expect_change, (b, i, t, expect_change)
    w.kv = base_kv


@pytest.mark.parametrize("fmt,h_q", [("bf16", 128), ("fp8", 16), ("bf16", 64)])
def test_invalid_page_ids_inside_a_sequence(fmt, h_q):
    """Block-table entries inside L that name no cache page (-1, or an id past
    the pool) mask their 64 tokens: the result matches the oracle (whose
    attended set skips them) and is the same bit for bit whichever invalid id
    is used. Positions past the block table's row are masked too."""
    from tests.gpu_helpers import compare, oracle, workload_floor_fn

    say(f"invalid page ids {fmt} h_q={h_q}")
    w = make_workload(batch=3, s_q=1, h_q=h_q, seqlens=[700, 300, 200], kv_format=fmt, extra_blocks=2, seed=32)
    w.block_table[0, 2] = -1
    w.block_table[0, 5] = w.num_blocks + 7
    w.block_table[1, 0] = -1            # the first page of a sequence
    w.block_table[2, 3] = -1            # its last, partly filled page
    a = run_gpu(w)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle(w)
    compare(a[0], a[1], o_ref, lse_ref, label="invalid page ids", floor_fn=workload_floor_fn(w))
    w.block_table[0, 2] = 1 << 30
    w.block_table[0, 5] = -5
    w.block_table[1, 0] = w.num_blocks
    w.block_table[2, 3] = -(1 << 30)
    b_ = run_gpu(w)
    torch.cuda.synchronize()
    assert _same(a, b_)
    # a block table of 3 pages: every sequence attends at most its first 192
    # tokens, as if L were 192 (one part, so both runs split alike)
    w.block_table = w.block_table[:, :3].contiguous()
    c = run_gpu(w, num_parts=1)
    torch.cuda.synchronize()
    w.cache_seqlens = torch.tensor([192, 192, 192], dtype=torch.int32)
    d = run_gpu(w, num_parts=1)
    torch.cuda.synchronize()
    assert _same(c, d)
    o_ref, lse_ref = oracle(w)
    compare(d[0], d[1], o_ref, lse_ref, label="positions past the block table", floor_fn=workload_floor_fn(w))


@pytest.mark.parametrize("fmt,h_q", [("bf16", 12), ("bf16", 40), ("fp8", 40), ("fp8_528", 12), ("bf16", 128)])
def test_causal_positions_past_the_block_table(fmt, h_q):
    """Causal calls with four query positions whose sequences run past their
    block-table row (3 pages, 192 tokens): position i attends its causal prefix
    cut at the row's end, so in one row group the early positions end inside
    the row and the later ones at its end (lengths 193 and 194), all end there
    (195, 300), or none does (130). Every query row matches the oracle, and
    widening the row with -1 pages changes nothing."""
    from tests.gpu_helpers import compare, oracle, workload_floor_fn

    say(f"causal positions past the block table {fmt} h_q={h_q}")
    lens = [193, 194, 195, 130, 300]
    w = make_workload(batch=5, s_q=4, h_q=h_q, seqlens=lens, kv_format=fmt, causal=True, extra_blocks=2, seed=33)
    w.block_table = w.block_table[:, :3].contiguous()
    a = run_gpu(w)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle(w)
    compare(a[0], a[1], o_ref, lse_ref, label="causal past the block table", floor_fn=workload_floor_fn(w))
    # widening the row with pages that name no cache page (-1) leaves the
    # attended set as it is, and the result the same bit for bit
    w.block_table = torch.cat([w.block_table, torch.full((5, 2), -1, dtype=torch.int32)], dim=1).contiguous()
    b_ = run_gpu(w)
    torch.cuda.synchronize()
    assert _same(a, b_)
