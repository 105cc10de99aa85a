"""The Python binding's argument checks, on the CPU: each malformed tensor is
named in a ValueError before any pointer reaches the library; a well-formed
set of CPU tensors is refused only because it is not on the GPU."""

import pytest
import torch

import mla_latent_kv_10_amd as m

B, S, H, NB, P = 2, 1, 16, 4, 8


def _valid(fp8=False, sparse=False):
    d = dict(
        q=torch.zeros(B, S, H, 576, dtype=torch.bfloat16),
        kv=torch.zeros(NB, 64, 656 if fp8 else 1152, dtype=torch.uint8),
        block_table=None if sparse else torch.zeros(B, 2, dtype=torch.int32),
        cache_seqlens=None if sparse else torch.zeros(B, dtype=torch.int32),
        tile_meta=torch.zeros(P, 8, dtype=torch.int32),
        split_offsets=torch.zeros(m.metadata_size(B, S, H, P)[1], dtype=torch.int32),
        softmax_scale=0.04, causal=False, is_fp8_kvcache=fp8,
        indices=torch.zeros(B, S, 64, dtype=torch.int32) if sparse else None,
        workspace=torch.zeros(m.workspace_size(B, S, H, P), dtype=torch.uint8),
        o=torch.zeros(B, S, H, 512, dtype=torch.bfloat16),
        lse=torch.zeros(B, S, H, dtype=torch.float32),
    )
    return d


@pytest.mark.parametrize("fp8,sparse", [(False, False), (True, False), (False, True), (True, True)])
def test_well_formed_cpu_tensors_are_refused_for_the_device_only(fp8, sparse):
    with pytest.raises(ValueError, match="on the GPU"):
        m.make_args(**_valid(fp8, sparse))


def test_bf16_cache_may_be_passed_as_bf16_values():
    d = _valid()
    d["kv"] = torch.zeros(NB, 64, 576, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on the GPU"):
        m.make_args(**d)


BAD = [
    ("q", lambda d: d["q"].float(), "q must be torch.bfloat16"),
    ("q", lambda d: torch.zeros(B, S, H, 512, dtype=torch.bfloat16), "q must have shape"),
    ("kv", lambda d: torch.zeros(NB, 64, 656, dtype=torch.uint8), "kv \\(bf16 cache as bytes\\) must have shape"),
    ("kv", lambda d: torch.zeros(NB, 32, 1152, dtype=torch.uint8), "must have shape"),
    ("block_table", lambda d: d["block_table"].long(), "block_table must be torch.int32"),
    ("block_table", lambda d: torch.zeros(B + 1, 2, dtype=torch.int32), "block_table must have shape"),
    ("cache_seqlens", lambda d: d["cache_seqlens"].long(), "cache_seqlens must be torch.int32"),
    ("cache_seqlens", lambda d: torch.zeros(B + 3, dtype=torch.int32), "cache_seqlens must have shape"),
    ("tile_meta", lambda d: torch.zeros(P, 4, dtype=torch.int32), "tile_meta must have shape"),
    ("split_offsets", lambda d: torch.zeros(B + 5, dtype=torch.int32), "split_offsets must have shape"),
    ("split_offsets", lambda d: d["split_offsets"].long(), "split_offsets must be torch.int32"),
    ("workspace", lambda d: d["workspace"].float(), "workspace must be torch.uint8"),
    ("o", lambda d: torch.zeros(B, S, H, 512, dtype=torch.float32), "o must be torch.bfloat16"),
    ("o", lambda d: torch.zeros(B, S, H - 1, 512, dtype=torch.bfloat16), "o must have shape"),
    ("lse", lambda d: torch.zeros(B, S, H, dtype=torch.bfloat16), "lse must be torch.float32"),
    ("lse", lambda d: torch.zeros(B, S, H + 1, dtype=torch.float32), "lse must have shape"),
]


@pytest.mark.parametrize("name,make,msg", BAD, ids=[f"{b[0]}-{i}" for i, b in enumerate(BAD)])
def test_each_malformed_tensor_is_named(name, make, msg):
    d = _valid()
    d[name] = make(d)
    with pytest.raises(ValueError, match=msg):
        m.make_args(**d)


def test_sparse_indices_must_be_int32_with_the_query_shape():
    d = _valid(sparse=True)
    d["indices"] = torch.zeros(B, S, 64, dtype=torch.int64)   # what torch.topk returns
    with pytest.raises(ValueError, match="indices must be torch.int32"):
        m.make_args(**d)
    d["indices"] = torch.zeros(B, S + 1, 64, dtype=torch.int32)
    with pytest.raises(ValueError, match="indices must have shape"):
        m.make_args(**d)


def test_fp8_cache_must_hold_656_byte_rows():
    d = _valid(fp8=True)
    d["kv"] = torch.zeros(NB, 64, 1152, dtype=torch.uint8)
    with pytest.raises(ValueError, match="FP8 cache"):
        m.make_args(**d)


def test_metadata_built_for_another_call_shape_is_refused():
    d = _valid()
    d["tile_meta"].mla_call_shape = (B, S, H, 64)   # built for a sparse call with topk 64
    with pytest.raises(ValueError, match="metadata was built for"):
        m.make_args(**d)
    d["tile_meta"].mla_call_shape = (B, S, H, 0)
    with pytest.raises(ValueError, match="on the GPU"):
        m.make_args(**d)


def test_library_shares_torchs_hip_runtime():
    """Loading the library before anything imports torch, then torch, leaves
    one HIP runtime in the process (torch's copy), not two."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import mla_latent_kv_10_amd as m\n"
            "m.lib()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(sorted({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n") % root
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    paths = eval(out.stdout.strip().splitlines()[-1])
    assert len(paths) == 1, paths
