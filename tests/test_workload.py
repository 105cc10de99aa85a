"""The seeded input generators: shapes, determinism and the stated workload recipes."""

import numpy as np
import pytest
import torch

from workload import config_workload, make_workload


def test_config1_shapes():
    w = config_workload(1)
    assert tuple(w.q.shape) == (1, 1, 4, 576) and w.q.dtype == torch.bfloat16
    assert tuple(w.kv.shape) == (4, 64, 1152) and w.kv.dtype == torch.uint8
    assert w.block_table.tolist()[0] != [0, 1, 2, 3] and sorted(w.block_table.tolist()[0]) == [0, 1, 2, 3]
    assert w.cache_seqlens.tolist() == [256]


def test_config2_recipe():
    w = config_workload(2)
    assert int(w.cache_seqlens.sum()) == 40165
    assert int(w.cache_seqlens.min()) >= 1024 and int(w.cache_seqlens.max()) <= 4096
    pages = [-(-int(l) // 64) for l in w.cache_seqlens]
    used = torch.cat([w.block_table[b, :n] for b, n in enumerate(pages)])
    assert sorted(used.tolist()) == list(range(w.num_blocks))
    for b, n in enumerate(pages):
        assert torch.all(w.block_table[b, n:] == -1)


def test_deterministic():
    a = make_workload(batch=2, s_q=2, h_q=8, seqlens=[70, 3], kv_format="fp8", causal=True, seed=5)
    b = make_workload(batch=2, s_q=2, h_q=8, seqlens=[70, 3], kv_format="fp8", causal=True, seed=5)
    assert torch.equal(a.q.view(torch.int16), b.q.view(torch.int16))
    assert torch.equal(a.kv, b.kv) and torch.equal(a.block_table, b.block_table)


def test_sparse_recipe_small():
    w = make_workload(batch=3, s_q=1, h_q=16, kv_format="fp8", topk=256, sparse_tokens_per_seq=1024,
                      invalid_frac=0.05, seed=0)
    assert w.block_table is None and tuple(w.indices.shape) == (3, 1, 256)
    for b in range(3):
        row = w.indices[b, 0]
        valid = row[row >= 0]
        assert int((row == -1).sum()) == round(0.05 * 256)
        assert len(set(valid.tolist())) == len(valid)
        assert int(valid.min()) >= b * 1024 and int(valid.max()) < (b + 1) * 1024


@pytest.mark.slow
def test_config5_recipe():
    w = config_workload(5)
    assert tuple(w.kv.shape) == (16384, 64, 656)
    assert torch.all((w.indices == -1).sum(dim=2) == 102)


def test_sparse_prefill_recipe():
    w = config_workload(6)
    assert w.q.shape == (1, 1024, 128, 576) and w.kv.shape == (512, 64, 1152) and w.indices.shape == (1, 1024, 2048)
    idx = w.indices.numpy()[0]
    T, s_q = 32768, 1024
    for i in (0, 1, 500, 1023):
        row = idx[i]
        assert row.min() >= 0 and row.max() <= T - s_q + i   # inside query i's visible prefix
        assert len(np.unique(row)) == row.size               # distinct
    assert not w.causal and w.block_table is None

