"""bench.py's host-side logic on the CPU: the algorithmic counts its roofline
uses, the lookup of the committed counter row, and the one-GPU guard."""

import os
import subprocess
import sys

import numpy as np

import bench
from workload import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_counts_dense_causal():
    w = make_workload(batch=3, s_q=2, h_q=8, seqlens=[5, 70, 1], kv_format="fp8", causal=True, seed=2, name="t")
    pairs, kv_bytes = bench.algorithmic_counts(w)
    # causal, bottom-right: query i of a length-L sequence attends min(L, max(0, L - s_q + 1 + i)) tokens
    attended = sum(max(0, L - 2 + 1 + i) for L in (5, 70, 1) for i in range(2))
    assert pairs == attended * 8
    assert kv_bytes == (5 + 70 + 1) * 656


def test_algorithmic_counts_sparse_distinct_rows():
    w = make_workload(batch=2, s_q=1, h_q=4, kv_format="bf16", topk=64, sparse_tokens_per_seq=128,
                      invalid_frac=0.25, seed=3, name="s")
    idx = w.indices.numpy()
    valid = (idx >= 0) & (idx < w.num_blocks * 64)
    pairs, kv_bytes = bench.algorithmic_counts(w)
    assert pairs == int(valid.sum()) * 4
    assert kv_bytes == sum(len(np.unique(idx[b][valid[b]])) for b in range(2)) * 1152


def test_committed_traffic_row_matches_the_kernel_sources():
    # the committed counter summary carries the hash of the current kernel sources
    got = bench.measured_traffic("dense bf16: B=16 s_q=1 h_q=128 L~U[1024,4096]", 256)
    assert got is not None and got > 46_270_080  # at least the KV bytes
    assert bench.measured_traffic("no such workload", 256) is None
    assert bench.measured_traffic("dense bf16: B=16 s_q=1 h_q=128 L~U[1024,4096]", 7) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_writer_traffic_row_and_cpu_leg():
    name, src, slots = bench.quantize_workload(batch=2, seqlen=4096)
    assert src.shape == (8192, 576) and sorted(slots.tolist()) == list(range(8192))
    # the committed writer row is keyed by the writer's own source hash
    full = "fp8 cache write: 524288 rows (64 x 8192 tokens) into 8192 shuffled pages"
    got = bench.measured_traffic(full, "-", bench.quantize_source_hash(), bench.QUANT_TRAFFIC_FILE)
    assert got is not None and got >= 524288 * bench.QUANT_ROW_BYTES
    assert bench.measured_traffic(full, "-", "0" * 16, bench.QUANT_TRAFFIC_FILE) is None
    leg = bench.quantize_cpu_baseline(src, 0.2)
    assert leg["kind"] == "oracle" and leg["unit"] == "GB/s" and leg["value"] > 0


def test_absorb_counts_and_traffic_rows():
    ba, bu, flops = bench.absorb_counts(128, 128)
    w = 128 * 128 * 512 * 2
    assert ba == w + 128 * 128 * (128 + 64 + 576) * 2 and bu == w + 128 * 128 * (512 + 128) * 2
    assert flops == 2 * 128 * 128 * 128 * 512
    name = "absorption products: T=128 tokens (B=64 x s_q=2), H=128"
    h = bench.source_hash(bench.ABSORB_SOURCES, "mla_absorb.hip")
    for kern, algo in (("absorb_q", ba), ("unabsorb_o", bu)):
        got = bench.measured_traffic(name, kern, h, bench.ABSORB_TRAFFIC_FILE)
        assert got is not None and algo <= got < 1.05 * algo
