"""HIP decode vs the float64 oracle on the same seeded inputs.

Every case, the six full-size workloads included, is compared on every query
row (b, i), in the launch configuration the benchmark uses (metadata with the
default number of parts, decode + combine). The cache sits between 64 KB NaN
guard bands on the GPU."""

import numpy as np
import pytest
import torch

from workload import config_workload, make_workload

from tests.gpu_helpers import compare, oracle, run_gpu, say, workload_floor_fn

pytestmark = pytest.mark.gpu


def _check(w, rows=None, num_parts=None, label=None):
    label = label or w.name
    say(f"case: {label} num_parts={num_parts}")
    o, lse, _, _ = run_gpu(w, num_parts=num_parts)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle(w, rows)
    return compare(o, lse, o_ref, lse_ref, rows, label, floor_fn=workload_floor_fn(w))


SMALL = [
    # (label, kwargs)
    ("bf16 dense h128 ragged", dict(batch=3, s_q=1, h_q=128, seqlens=[1, 130, 700], kv_format="bf16")),
    ("bf16 dense h16 ragged", dict(batch=4, s_q=1, h_q=16, seqlens=[64, 65, 1000, 3], kv_format="bf16")),
    ("bf16 dense h4", dict(batch=2, s_q=1, h_q=4, seqlens=[256, 77], kv_format="bf16")),
    ("bf16 dense h20 64-head group", dict(batch=2, s_q=1, h_q=20, seqlens=[300, 129], kv_format="bf16")),
    ("bf16 dense h64", dict(batch=3, s_q=1, h_q=64, seqlens=[1000, 1, 64], kv_format="bf16")),
    ("fp8 causal h48 s_q=2", dict(batch=2, s_q=2, h_q=48, seqlens=[700, 33], kv_format="fp8", causal=True)),
    ("fp8 sparse h64", dict(batch=2, s_q=1, h_q=64, kv_format="fp8", topk=300, sparse_tokens_per_seq=1024,
                            invalid_frac=0.05)),
    ("bf16 dense h100 padded rows", dict(batch=2, s_q=1, h_q=100, seqlens=[200, 513], kv_format="bf16")),
    ("bf16 dense h130 two row groups", dict(batch=1, s_q=1, h_q=130, seqlens=[333], kv_format="bf16")),
    ("bf16 dense empty sequence", dict(batch=3, s_q=1, h_q=128, seqlens=[0, 100, 0], kv_format="bf16")),
    ("bf16 causal s_q=3", dict(batch=2, s_q=3, h_q=16, seqlens=[200, 2], kv_format="bf16", causal=True)),
    ("bf16 causal s_q=2 h128", dict(batch=2, s_q=2, h_q=128, seqlens=[129, 64], kv_format="bf16", causal=True)),
    ("fp8 dense h128", dict(batch=2, s_q=1, h_q=128, seqlens=[500, 64], kv_format="fp8")),
    ("fp8 dense h16", dict(batch=3, s_q=1, h_q=16, seqlens=[1, 190, 640], kv_format="fp8")),
    ("fp8 causal s_q=2 h128", dict(batch=3, s_q=2, h_q=128, seqlens=[1000, 65, 1], kv_format="fp8", causal=True)),
    ("fp8 sparse h128", dict(batch=3, s_q=1, h_q=128, kv_format="fp8", topk=200, sparse_tokens_per_seq=1024,
                             invalid_frac=0.05)),
    ("fp8 sparse h16 s_q=2", dict(batch=2, s_q=2, h_q=16, kv_format="fp8", topk=130, sparse_tokens_per_seq=512,
                                  invalid_frac=0.1)),
    # FP8 with 128 heads: short segments (tile loads past a segment's end,
    # parts that span several sequences) and the sparse index ring
    ("fp8 dense h128 short sequences", dict(batch=6, s_q=1, h_q=128, seqlens=[1, 65, 129, 2, 64, 300], kv_format="fp8")),
    ("fp8 sparse h128 s_q=2", dict(batch=3, s_q=2, h_q=128, kv_format="fp8", topk=130, sparse_tokens_per_seq=704,
                                   invalid_frac=0.1)),
    ("bf16 sparse h128", dict(batch=2, s_q=1, h_q=128, kv_format="bf16", topk=256, sparse_tokens_per_seq=2048,
                              invalid_frac=0.05)),
    ("bf16 sparse h4 mostly invalid", dict(batch=2, s_q=1, h_q=4, kv_format="bf16", topk=100,
                                           sparse_tokens_per_seq=256, invalid_frac=0.95)),
    ("bf16 sparse h48 s_q=2", dict(batch=2, s_q=2, h_q=48, kv_format="bf16", topk=300, sparse_tokens_per_seq=1024,
                                   invalid_frac=0.1)),
    ("bf16 dense h32 ragged", dict(batch=3, s_q=1, h_q=32, seqlens=[1, 700, 129], kv_format="bf16")),
    ("bf16 sparse prefill chunk h128 s_q=40", dict(batch=2, s_q=40, h_q=128, kv_format="bf16", topk=192,
                                                   sparse_tokens_per_seq=512, prefix_sparse=True)),
    ("fp8 sparse prefill chunk h16 s_q=33", dict(batch=1, s_q=33, h_q=16, kv_format="fp8", topk=100,
                                                 sparse_tokens_per_seq=256, prefix_sparse=True, invalid_frac=0.1)),
    # dense calls pack all s_q * h_q rows of a sequence into one row space:
    # row groups that hold several positions (each with its own causal limit),
    # positions cut across row-group boundaries, a position with no token
    ("bf16 causal s_q=2 h16 packed, L < s_q", dict(batch=3, s_q=2, h_q=16, seqlens=[1, 2, 300], kv_format="bf16",
                                                    causal=True)),
    ("bf16 causal s_q=8 h16 packed 128 rows", dict(batch=3, s_q=8, h_q=16, seqlens=[64, 65, 63], kv_format="bf16",
                                                    causal=True)),
    ("fp8 causal s_q=2 h64 packed", dict(batch=2, s_q=2, h_q=64, seqlens=[700, 129], kv_format="fp8", causal=True)),
    ("bf16 causal s_q=3 h100 positions across groups", dict(batch=2, s_q=3, h_q=100, seqlens=[190, 5],
                                                              kv_format="bf16", causal=True)),
    ("bf16 dense s_q=2 h16 packed, not causal", dict(batch=2, s_q=2, h_q=16, seqlens=[640, 77], kv_format="bf16")),
    ("fp8_528 causal s_q=5 h4 packed", dict(batch=2, s_q=5, h_q=4, seqlens=[260, 4], kv_format="fp8_528",
                                            causal=True)),
    # position-spanning row groups in every format and row-group size
    ("bf16 causal s_q=4 h4 packed 16 rows", dict(batch=2, s_q=4, h_q=4, seqlens=[333, 3], kv_format="bf16",
                                                 causal=True)),
    ("fp8 causal s_q=2 h8 packed 16 rows", dict(batch=2, s_q=2, h_q=8, seqlens=[129, 64], kv_format="fp8",
                                                causal=True)),
    ("fp8 causal s_q=3 h16 packed 48 rows", dict(batch=2, s_q=3, h_q=16, seqlens=[500, 66], kv_format="fp8",
                                                 causal=True)),
    ("fp8_528 causal s_q=3 h5 packed 15 rows", dict(batch=2, s_q=3, h_q=5, seqlens=[191, 2], kv_format="fp8_528",
                                                    causal=True)),
    ("fp8_528 causal s_q=2 h96 packed 192 rows", dict(batch=2, s_q=2, h_q=96, seqlens=[450, 128],
                                                      kv_format="fp8_528", causal=True)),
    # one head, many positions: every row its own causal limit; with L < s_q the
    # first rows of the group see no token at all (o = 0, lse = -inf)
    ("bf16 causal s_q=20 h1 packed", dict(batch=2, s_q=20, h_q=1, seqlens=[300, 129], kv_format="bf16",
                                          causal=True)),
    ("fp8 causal s_q=100 h1 packed, L < s_q", dict(batch=2, s_q=100, h_q=1, seqlens=[50, 700], kv_format="fp8",
                                                   causal=True)),
    ("bf16 causal s_q=3 h5 packed, L < s_q", dict(batch=3, s_q=3, h_q=5, seqlens=[1, 2, 40], kv_format="bf16",
                                                  causal=True)),
    ("fp8_528 causal s_q=4 h12 packed, L < s_q", dict(batch=4, s_q=4, h_q=12, seqlens=[1, 2, 3, 200],
                                                      kv_format="fp8_528", causal=True)),
    # 528-byte rows: 512-dim keys, 448-dim values, UE8M0 scales per 32 values
    ("fp8_528 dense h128 ragged", dict(batch=3, s_q=1, h_q=128, seqlens=[1, 130, 700], kv_format="fp8_528")),
    ("fp8_528 dense h16 ragged", dict(batch=4, s_q=1, h_q=16, seqlens=[64, 65, 1000, 3], kv_format="fp8_528")),
    ("fp8_528 dense h64", dict(batch=3, s_q=1, h_q=64, seqlens=[1000, 1, 64], kv_format="fp8_528")),
    ("fp8_528 causal s_q=2 h128", dict(batch=3, s_q=2, h_q=128, seqlens=[1000, 65, 1], kv_format="fp8_528",
                                       causal=True)),
    ("fp8_528 causal s_q=3 h20", dict(batch=2, s_q=3, h_q=20, seqlens=[300, 2], kv_format="fp8_528", causal=True)),
    ("fp8_528 empty sequence h128", dict(batch=3, s_q=1, h_q=128, seqlens=[0, 100, 0], kv_format="fp8_528")),
    ("fp8_528 sparse h128", dict(batch=3, s_q=1, h_q=128, kv_format="fp8_528", topk=200, sparse_tokens_per_seq=1024,
                                 invalid_frac=0.05)),
    ("fp8_528 sparse h128 s_q=2", dict(batch=3, s_q=2, h_q=128, kv_format="fp8_528", topk=130,
                                       sparse_tokens_per_seq=704, invalid_frac=0.1)),
    ("fp8_528 sparse h16 s_q=2", dict(batch=2, s_q=2, h_q=16, kv_format="fp8_528", topk=130,
                                      sparse_tokens_per_seq=512, invalid_frac=0.1)),
    ("fp8_528 sparse h64", dict(batch=2, s_q=1, h_q=64, kv_format="fp8_528", topk=300, sparse_tokens_per_seq=1024,
                                invalid_frac=0.05)),
]


@pytest.mark.parametrize("label,kw", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("num_parts", [None, 1, 7])
def test_small_cases(label, kw, num_parts):
    w = make_workload(seed=11, name=label, **kw)
    _check(w, num_parts=num_parts, label=f"{label} parts={num_parts}")


def test_sparse_all_invalid_rows():
    w = make_workload(batch=2, s_q=1, h_q=128, kv_format="fp8", topk=64, sparse_tokens_per_seq=256,
                      invalid_frac=0.0, seed=3, name="all -1")
    w.indices[0] = -1
    w.indices[1, 0, 5] = 10 ** 9        # out of range counts as unused
    w.indices[1, 0, 6] = -7
    _check(w, label="sparse all -1 / out of range")


def test_config1_tiny():
    _check(config_workload(1), label="config 1 (tiny dense)")


def test_config2_dense_bf16_full():
    w = config_workload(2)
    _check(w, label="config 2 (dense bf16, all rows)")


@pytest.mark.parametrize("L", [512, 1024, 2048, 4096, 8192, 16384, 32768, 65536])
def test_config3_low_head_all_rows(L):
    _check(config_workload(3, seqlen=L), label=f"config 3 L={L} (all rows)")


def test_config4_fp8_causal_all_rows():
    _check(config_workload(4), label="config 4 (fp8 causal, all rows)")


def test_config5_sparse_fp8_all_rows():
    _check(config_workload(5), label="config 5 (sparse fp8, all rows)")


def test_config6_sparse_prefill_all_rows():
    _check(config_workload(6), label="config 6 (sparse prefill, all rows)")


def test_config7_64_head_share_all_rows():
    _check(config_workload(7), label="config 7 (dense bf16, 64 heads, all rows)")


def test_config8_fp8_528_causal_all_rows():
    _check(config_workload(8), label="config 8 (528-byte rows, causal, all rows)")


def test_config9_sparse_fp8_528_all_rows():
    _check(config_workload(9), label="config 9 (528-byte rows, sparse, all rows)")


def test_config10_two_position_low_head_all_rows():
    _check(config_workload(10), label="config 10 (two positions packed, causal, all rows)")
