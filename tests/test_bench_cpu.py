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


def test_traffic_lookup(tmp_path):
    f = tmp_path / "t.md"
    f.write_text("| traffic | w a | 256 | 1000 | abcd |\n| traffic | w b | 256 | 2000 | ffff |\n")
    assert bench.measured_traffic("w a", 256, "abcd", str(f)) == 1000
    assert bench.measured_traffic("w a", 256, "ffff", str(f)) is None      # the kernel changed since
    assert bench.measured_traffic("w a", 7, "abcd", str(f)) is None
    assert bench.measured_traffic("no such workload", 256, "abcd", str(f)) is None


def test_committed_traffic_rows_cover_the_kv_bytes():
    """Every committed counter row of a decode workload reads at least that
    workload's algorithmic KV bytes (HBM traffic cannot be below them)."""
    from workload import CONFIG_NAMES, config_workload

    names = {v: k for k, v in CONFIG_NAMES.items()}
    rows = 0
    for line in open(bench.TRAFFIC_FILE, encoding="utf-8"):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) != 5 or cells[0] != "traffic":
            continue
        name = cells[1]
        cfg, L = names.get(name), None
        if cfg is None and name.startswith(CONFIG_NAMES[3] + " L="):
            cfg, L = 3, int(name.rsplit("=", 1)[1])
        if cfg is None or (cfg == 3 and L > 16384):
            continue  # only workloads cheap to build on the CPU here
        w = config_workload(cfg, seqlen=L or 8192)
        _, kv_bytes = bench.algorithmic_counts(w)
        assert int(cells[3]) >= kv_bytes, (name, cells[3], kv_bytes)
        rows += 1
    assert rows >= 1


def test_roofline_bound_follows_the_ridge():
    # below 2.5 PFLOP/s / 8 TB/s = 312.5 FLOP per KV byte: HBM; above: bf16 MFMA
    r = bench.roofline_entry(flops=300 * 10**9, kv_bytes=10**9, kernel_ms=1.0, traffic=None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and abs(r["achieved"] - 1000.0) < 1e-6
    assert abs(r["frac"] - 0.125) < 1e-9
    r = bench.roofline_entry(flops=400 * 10**9, kv_bytes=10**9, kernel_ms=1.0, traffic=123)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and abs(r["achieved"] - 400.0) < 1e-6
    assert r["traffic"] == 123 and r["per_launch"] == {"flop": 400 * 10**9, "kv_bytes": 10**9}
    assert isinstance(bench.cpu_model(), str)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_writer_traffic_row_and_cpu_leg():
    name, src, slots = bench.quantize_workload(batch=2, seqlen=4096)
    assert src.shape == (8192, 576) and sorted(slots.tolist()) == list(range(8192))
    # the committed writer row (keyed by the writer's own source hash) covers the algorithmic bytes
    full = "fp8 cache write: 524288 rows (64 x 8192 tokens) into 8192 shuffled pages"
    row = [[c.strip() for c in ln.strip().strip("|").split("|")] for ln in open(bench.QUANT_TRAFFIC_FILE, encoding="utf-8")]
    row = [r for r in row if len(r) == 5 and r[0] == "traffic" and r[1] == full]
    assert len(row) == 1 and int(row[0][3]) >= 524288 * bench.QUANT_ROW_BYTES
    assert bench.measured_traffic(full, "-", "0" * 16, bench.QUANT_TRAFFIC_FILE) is None
    leg = bench.quantize_cpu_baseline(src, 0.2)
    assert leg["kind"] == "oracle" and leg["unit"] == "GB/s" and leg["value"] > 0


def test_absorb_counts_and_traffic_rows():
    ba, bu, flops = bench.absorb_counts(128, 128)
    w = 128 * 128 * 512 * 2
    assert ba == w + 128 * 128 * (128 + 64 + 576) * 2 and bu == w + 128 * 128 * (512 + 128) * 2
    assert flops == 2 * 128 * 128 * 128 * 512
    name = "absorption products: T=128 tokens (B=64 x s_q=2), H=128"
    rows = [[c.strip() for c in ln.strip().strip("|").split("|")] for ln in open(bench.ABSORB_TRAFFIC_FILE, encoding="utf-8")]
    rows = {r[2]: int(r[3]) for r in rows if len(r) == 5 and r[0] == "traffic" and r[1] == name}
    for kern, algo in (("absorb_q", ba), ("unabsorb_o", bu)):
        assert algo <= rows[kern] < 1.05 * algo


def test_source_hash_ignores_comments_only():
    """The kernel sources hash keys the committed counter rows: an edit to comments or blank lines
    keeps it, any change to the code (string literals included) moves it."""
    code = 'int a = 1; // note\n/* block\n comment */ const char* s = "x // y /* z */";\n\nint b;\n'
    same = '// header\nint a = 1;\n\n  const char* s = "x // y /* z */";   // trailing\nint b;'
    assert bench.code_without_comments(code) == bench.code_without_comments(same)
    assert bench.code_without_comments(code) != bench.code_without_comments(code.replace("b;", "c;"))
    assert bench.code_without_comments(code) != bench.code_without_comments(code.replace("// y", "// w"))
    assert bench.code_without_comments("char c = '\\'';  // q\nint d;") == "char c = '\\'';\nint d;"


def test_fractions_against_the_measured_peaks():
    peaks = {"hbm_read_GBps": 7000.0, "mfma_bf16_TFLOPS": 2450.0}
    out = {"roofline": {"bound": "hbm", "achieved": 3500.0},
           "sweep": [{"roofline": {"bound": "hbm", "achieved": 700.0}}],
           "configs": {"a": {"roofline": {"bound": "mfma", "achieved": 980.0}}},
           "ops": {"q": {"roofline": {"bound": "hbm", "achieved": 1400.0}}}}
    bench.add_achievable_fracs(out, peaks)
    assert out["roofline"]["frac_of_achievable"] == 0.5
    assert out["sweep"][0]["roofline"]["frac_of_achievable"] == 0.1
    assert out["configs"]["a"]["roofline"]["frac_of_achievable"] == 0.4
    assert out["ops"]["q"]["roofline"]["frac_of_achievable"] == 0.2
