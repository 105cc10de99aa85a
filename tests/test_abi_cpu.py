"""The C ABI on the CPU: the library loads, exports what include/mla.h declares,
its argument block matches the header, and every argument error is reported
before any HIP call (no GPU is touched by these tests)."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import mla_latent_kv_10_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = m.lib()
    declared = _declared_functions()
    assert declared == sorted(m.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_every_export_declares_argument_types():
    # without argtypes ctypes passes a Python int as a 32-bit C int, which
    # truncates device pointers and stream handles
    L = m.lib()
    for name in m.EXPORTS:
        assert getattr(L, name).argtypes is not None, name


def test_argument_block_layout_matches_header():
    fields = [f for f, _ in m.MlaDecodeArgs._fields_]
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"mla.h\"\nint main(void){\n"
    src += 'printf("%zu\\n", sizeof(mla_decode_args));\n'
    for f in fields:
        src += f'printf("%zu\\n", offsetof(mla_decode_args, {f}));\n'
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        out = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(m.MlaDecodeArgs)
    for f, off in zip(fields, out[1:]):
        assert getattr(m.MlaDecodeArgs, f).offset == off, f


def test_sizes():
    # h_q = 128: row groups of 128; s_q = 2 -> Q = 2 * batch units
    assert m.metadata_size(64, 2, 128, 256) == (256 * 8, 64 * 2 + 1)
    # h_q = 16: row groups of 16
    assert m.metadata_size(16, 1, 16, 256) == (256 * 8, 17)
    # 16 < h_q <= 64: 64-head groups
    assert m.metadata_size(16, 1, 40, 256) == (256 * 8, 16 + 1)
    # fp16 partial rows, then fp32 lse and fp32 scale per (slot, row)
    ws = m.workspace_size(16, 1, 64, 256)
    slots = 16 + 256
    assert ws == ((slots * 64 * 512 * 2 + 255) // 256) * 256 + 2 * slots * 64 * 4
    ws = m.workspace_size(64, 1, 128, 256)
    slots = 64 + 256
    assert ws == ((slots * 128 * 512 * 2 + 255) // 256) * 256 + 2 * slots * 128 * 4


def _ws(slots, rg):
    return ((slots * rg * 512 * 2 + 255) // 256) * 256 + 2 * slots * rg * 4


def test_sizes_cover_dense_and_sparse_row_spaces():
    # s_q = 2, h_q = 16: a dense call packs 32 rows per sequence (one 64-row
    # group); a sparse call has two 16-row groups, one per position
    assert m.metadata_size(16, 2, 16, 256) == (256 * 8, 16 * 2 + 1)
    assert m.workspace_size(16, 2, 16, 256) == max(_ws(16 + 256, 64), _ws(32 + 256, 16))
    # s_q = 4, h_q = 32: dense 128 rows = one 128-row group; sparse 4 x one 64-row group
    assert m.metadata_size(8, 4, 32, 64) == (64 * 8, 8 * 4 + 1)
    assert m.workspace_size(8, 4, 32, 64) == max(_ws(8 + 64, 128), _ws(32 + 64, 64))
    # the sparse shape exceeds the unit limit (4096 x 4 groups), the dense one fits:
    # the sizes are the dense call's
    assert m.metadata_size(4096, 4, 16, 256) == (256 * 8, 4096 + 1)
    assert m.workspace_size(4096, 4, 16, 256) == _ws(4096 + 256, 64)


@pytest.mark.parametrize("bad", [dict(batch=0), dict(s_q=0), dict(h_q=0), dict(num_parts=0), dict(num_parts=70000)])
def test_size_queries_reject_bad_shapes(bad):
    kw = dict(batch=4, s_q=1, h_q=128, num_parts=256)
    kw.update(bad)
    with pytest.raises(m.MlaError) as e:
        m.workspace_size(**kw)
    assert e.value.status == m.MLA_ERR_INVALID


def test_too_many_units_is_unsupported():
    with pytest.raises(m.MlaError) as e:
        m.metadata_size(9000, 1, 128, 256)
    assert e.value.status == m.MLA_ERR_UNSUPPORTED


FAKE = 0x100000  # a 256-aligned non-null address; never dereferenced (validation fails first)


def _args(**over):
    a = m.MlaDecodeArgs()
    a.struct_size = ctypes.sizeof(m.MlaDecodeArgs)
    a.batch, a.s_q, a.h_q = 2, 1, 128
    a.q = a.kv = a.o = a.lse = FAKE
    a.num_blocks = 4
    a.block_size = 64
    a.row_bytes = 1152
    a.kv_format = m.MLA_KV_BF16
    a.block_table = a.cache_seqlens = FAKE
    a.max_blocks_per_seq = 2
    a.indices = 0
    a.topk = 0
    a.softmax_scale = 576 ** -0.5
    a.causal = 0
    a.tile_meta = a.split_offsets = FAKE
    a.num_parts = 8
    a.workspace = FAKE
    a.workspace_bytes = m.workspace_size(2, 1, 128, 8)
    for k, v in over.items():
        setattr(a, k, v)
    return a


CASES = [
    (dict(struct_size=8), m.MLA_ERR_INVALID, "struct_size"),
    (dict(q=0), m.MLA_ERR_INVALID, "non-NULL"),
    (dict(o=FAKE + 4), m.MLA_ERR_INVALID, "aligned"),
    (dict(block_size=32), m.MLA_ERR_UNSUPPORTED, "block_size"),
    (dict(kv_format=7), m.MLA_ERR_INVALID, "kv_format"),
    (dict(kv_format=m.MLA_KV_FP8_656), m.MLA_ERR_INVALID, "row_bytes"),       # bf16 rows flagged fp8
    (dict(row_bytes=656), m.MLA_ERR_INVALID, "row_bytes"),                    # fp8 rows flagged bf16
    (dict(num_blocks=0), m.MLA_ERR_INVALID, "num_blocks"),
    (dict(num_blocks=1 << 26), m.MLA_ERR_UNSUPPORTED, "2^31"),
    (dict(num_blocks=(1 << 32) // (64 * 1152) + 1), m.MLA_ERR_UNSUPPORTED, "4 GiB"),
    (dict(num_blocks=(1 << 32) // (64 * 656) + 1, kv_format=m.MLA_KV_FP8_656, row_bytes=656),
     m.MLA_ERR_UNSUPPORTED, "4 GiB"),
    (dict(indices=FAKE, topk=0, block_table=0, cache_seqlens=0), m.MLA_ERR_INVALID, "topk"),
    (dict(indices=FAKE, topk=64, causal=1), m.MLA_ERR_INVALID, "causal"),
    (dict(block_table=0), m.MLA_ERR_INVALID, "block_table"),
    (dict(max_blocks_per_seq=0), m.MLA_ERR_INVALID, "max_blocks_per_seq"),
    (dict(topk=5), m.MLA_ERR_INVALID, "topk"),
    (dict(softmax_scale=float("nan")), m.MLA_ERR_INVALID, "softmax_scale"),
    (dict(tile_meta=0), m.MLA_ERR_INVALID, "tile_meta"),
    (dict(workspace=0), m.MLA_ERR_INVALID, "workspace"),
    (dict(workspace=FAKE + 16), m.MLA_ERR_INVALID, "256-byte"),
    (dict(workspace_bytes=16), m.MLA_ERR_WORKSPACE, "workspace_bytes"),
    (dict(batch=0), m.MLA_ERR_INVALID, "batch"),
    (dict(h_q=0), m.MLA_ERR_INVALID, "h_q"),
    (dict(indices=FAKE, topk=(1 << 23) + 1, block_table=0, cache_seqlens=0), m.MLA_ERR_UNSUPPORTED, "2^23"),
    (dict(batch=64, indices=FAKE, topk=1 << 23, block_table=0, cache_seqlens=0), m.MLA_ERR_UNSUPPORTED, "2^29"),
    (dict(max_blocks_per_seq=(1 << 17) + 1), m.MLA_ERR_UNSUPPORTED, "2^17"),
    (dict(q=FAKE + 8), m.MLA_ERR_INVALID, "aligned"),
    (dict(kv=FAKE + 4), m.MLA_ERR_INVALID, "aligned"),
    (dict(lse=FAKE + 2), m.MLA_ERR_INVALID, "aligned"),
    (dict(tile_meta=FAKE + 4), m.MLA_ERR_INVALID, "tile_meta must be 16-byte aligned"),
    (dict(split_offsets=FAKE + 2), m.MLA_ERR_INVALID, "split_offsets 4-byte aligned"),
    (dict(block_table=FAKE + 2), m.MLA_ERR_INVALID, "4-byte aligned"),
    (dict(cache_seqlens=FAKE + 1), m.MLA_ERR_INVALID, "4-byte aligned"),
    (dict(indices=FAKE + 2, topk=64, block_table=0, cache_seqlens=0), m.MLA_ERR_INVALID, "indices must be 4-byte"),
]


@pytest.mark.parametrize("over,status,word", CASES)
def test_decode_argument_errors(over, status, word):
    L = m.lib()
    a = _args(**over)
    for fn in (L.mla_decode_with_kvcache, L.mla_decode_splits, L.mla_combine):
        rc = fn(ctypes.byref(a), None)
        msg = L.mla_last_error().decode()
        if fn is L.mla_combine and rc == status:
            assert word in msg
        if fn is not L.mla_combine:
            assert rc == status, msg
            assert word in msg, msg


def test_null_args_and_metadata_errors():
    L = m.lib()
    assert L.mla_decode_with_kvcache(None, None) == m.MLA_ERR_INVALID
    assert L.mla_decode_splits(None, None) == m.MLA_ERR_INVALID
    assert L.mla_get_metadata(FAKE, 4, 1, 128, -1, 256, FAKE, FAKE, None) == m.MLA_ERR_INVALID
    assert L.mla_get_metadata(0, 4, 1, 128, 0, 256, FAKE, FAKE, None) == m.MLA_ERR_INVALID
    assert L.mla_get_metadata(FAKE, 4, 1, 128, 0, 256, 0, FAKE, None) == m.MLA_ERR_INVALID
    assert L.mla_get_metadata(FAKE, 4, 1, 128, 0, 0, FAKE, FAKE, None) == m.MLA_ERR_INVALID
    assert b"num_parts" in L.mla_last_error()
    assert L.mla_get_metadata(FAKE, 4, 1, 128, (1 << 23) + 1, 256, FAKE, FAKE, None) == m.MLA_ERR_UNSUPPORTED
    assert b"2^23" in L.mla_last_error()
    # misaligned buffers: a scalar load ignores an address's low bits, so they are refused
    assert L.mla_get_metadata(FAKE + 2, 4, 1, 128, 0, 256, FAKE, FAKE, None) == m.MLA_ERR_INVALID
    assert b"cache_seqlens must be 4-byte aligned" in L.mla_last_error()
    assert L.mla_get_metadata(FAKE, 4, 1, 128, 0, 256, FAKE + 8, FAKE, None) == m.MLA_ERR_INVALID
    assert b"tile_meta must be 16-byte aligned" in L.mla_last_error()
    assert L.mla_get_metadata(FAKE, 4, 1, 128, 0, 256, FAKE, FAKE + 2, None) == m.MLA_ERR_INVALID
    assert b"split_offsets 4-byte aligned" in L.mla_last_error()
    # a sparse call reads no lengths: their pointer is not checked
    assert L.mla_get_metadata(FAKE + 2, 4, 1, 128, 64, 256, FAKE + 8, FAKE, None) == m.MLA_ERR_INVALID
    assert b"tile_meta" in L.mla_last_error()


QUANT_CASES = [
    (dict(n=-1), m.MLA_ERR_INVALID, "n must be"),
    (dict(n=1 << 31), m.MLA_ERR_UNSUPPORTED, "2^31"),
    (dict(num_blocks=0), m.MLA_ERR_INVALID, "num_blocks"),
    (dict(num_blocks=1 << 26), m.MLA_ERR_UNSUPPORTED, "2^31"),
    (dict(src=0), m.MLA_ERR_INVALID, "non-NULL"),
    (dict(slots=0), m.MLA_ERR_INVALID, "non-NULL"),
    (dict(kv=0), m.MLA_ERR_INVALID, "non-NULL"),
    (dict(src=FAKE + 8), m.MLA_ERR_INVALID, "aligned"),
    (dict(kv=FAKE + 4), m.MLA_ERR_INVALID, "aligned"),
    (dict(slots=FAKE + 2), m.MLA_ERR_INVALID, "aligned"),
]


@pytest.mark.parametrize("over,status,text", QUANT_CASES)
def test_quantize_rejects_bad_arguments(over, status, text):
    kw = dict(src=FAKE, slots=FAKE, n=8, kv=FAKE, num_blocks=4)
    kw.update(over)
    st = m.lib().mla_quantize_fp8_append(kw["src"], kw["slots"], kw["n"], kw["kv"], kw["num_blocks"], None)
    assert st == status
    assert text in m.lib().mla_last_error().decode()


def test_quantize_with_no_rows_enqueues_nothing():
    # n == 0 returns before any HIP call, so it succeeds without a GPU and with NULL buffers
    assert m.lib().mla_quantize_fp8_append(0, 0, 0, 0, 4, None) == m.MLA_OK


ABSORB_CASES = [
    (dict(tokens=-1), m.MLA_ERR_INVALID, "tokens"),
    (dict(heads=0), m.MLA_ERR_INVALID, "heads"),
    (dict(heads=5000), m.MLA_ERR_UNSUPPORTED, "heads"),
    (dict(tokens=1 << 31), m.MLA_ERR_UNSUPPORTED, "2^31"),
    (dict(x=0), m.MLA_ERR_INVALID, "non-NULL"),
    (dict(w=0), m.MLA_ERR_INVALID, "non-NULL"),
    (dict(out=0), m.MLA_ERR_INVALID, "non-NULL"),
    (dict(x=FAKE + 8), m.MLA_ERR_INVALID, "aligned"),
    (dict(w=FAKE + 2), m.MLA_ERR_INVALID, "aligned"),
    (dict(out=FAKE + 4), m.MLA_ERR_INVALID, "aligned"),
]


@pytest.mark.parametrize("over,status,text", ABSORB_CASES)
def test_absorb_entry_points_reject_bad_arguments(over, status, text):
    kw = dict(x=FAKE, w=FAKE, out=FAKE, tokens=8, heads=16)
    kw.update(over)
    L = m.lib()
    assert L.mla_absorb_q(kw["x"], FAKE, kw["w"], kw["tokens"], kw["heads"], kw["out"], None) == status
    assert text in L.mla_last_error().decode()
    assert L.mla_unabsorb_o(kw["x"], kw["w"], kw["tokens"], kw["heads"], kw["out"], None) == status
    assert text in L.mla_last_error().decode()


def test_absorb_rope_pointer_is_checked():
    assert m.lib().mla_absorb_q(FAKE, 0, FAKE, 8, 16, FAKE, None) == m.MLA_ERR_INVALID
    assert m.lib().mla_absorb_q(FAKE, FAKE + 8, FAKE, 8, 16, FAKE, None) == m.MLA_ERR_INVALID


@pytest.mark.parametrize("over,status,word", [c for c in CASES if not any(k.startswith("workspace") for k in c[0])])
def test_static_entry_checks_arguments_first(over, status, word):
    # every argument check runs on the host before the scratch is looked up
    L = m.lib()
    rc = L.mla_decode_with_kvcache_static(ctypes.byref(_args(**over)), None)
    assert rc == status and word in L.mla_last_error().decode()


def test_static_entry_refuses_shapes_beyond_its_scratch():
    L = m.lib()
    assert L.mla_decode_with_kvcache_static(None, None) == m.MLA_ERR_INVALID
    # 1024 query positions x 128 heads: 1280 split slots of 128 KB, more than 64 MiB
    a = _args(batch=1, s_q=1024, num_parts=256)
    assert m.workspace_size(1, 1024, 128, 256) > 64 << 20
    assert L.mla_decode_with_kvcache_static(ctypes.byref(a), None) == m.MLA_ERR_UNSUPPORTED
    assert "static scratch" in L.mla_last_error().decode()
    # the workspace fields are ignored: a NULL workspace is not the error reported
    a = _args(workspace=0, workspace_bytes=0, batch=1, s_q=1024, num_parts=256)
    assert L.mla_decode_with_kvcache_static(ctypes.byref(a), None) == m.MLA_ERR_UNSUPPORTED


PROBE_MFMA_CASES = [
    (dict(iters=0), "iters"),
    (dict(blocks=0), "blocks"),
    (dict(blocks=(1 << 20) + 1), "blocks"),
    (dict(sink=0), "sink"),
    (dict(sink=FAKE + 2), "sink"),
]


@pytest.mark.parametrize("over,text", PROBE_MFMA_CASES)
def test_mfma_probe_rejects_bad_arguments(over, text):
    kw = dict(iters=10, blocks=4, sink=FAKE)
    kw.update(over)
    assert m.lib().mla_probe_mfma_bf16(kw["iters"], kw["blocks"], 1.0, kw["sink"], None) == m.MLA_ERR_INVALID
    assert text in m.lib().mla_last_error().decode()


PROBE_READ_CASES = [
    (dict(nbytes=0), "multiple of 16"),
    (dict(nbytes=24), "multiple of 16"),
    (dict(blocks=0), "blocks"),
    (dict(src=0), "non-NULL"),
    (dict(src=FAKE + 8), "aligned"),
    (dict(sink=0), "non-NULL"),
    (dict(sink=FAKE + 1), "aligned"),
]


@pytest.mark.parametrize("over,text", PROBE_READ_CASES)
def test_read_probe_rejects_bad_arguments(over, text):
    kw = dict(src=FAKE, nbytes=4096, blocks=4, sink=FAKE)
    kw.update(over)
    assert m.lib().mla_probe_hbm_read(kw["src"], kw["nbytes"], kw["blocks"], kw["sink"], None) == m.MLA_ERR_INVALID
    assert text in m.lib().mla_last_error().decode()
