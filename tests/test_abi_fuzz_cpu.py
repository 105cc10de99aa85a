"""Randomised checks of the C ABI's host validation, written from the contract
in include/mla.h (no GPU is used).

A call that the header documents as valid passes validation and fails only
where the library first touches the GPU (MLA_ERR_HIP on a host without one);
the same call with one field broken as the header describes fails with the
status the header gives, before any HIP call. Skipped where a GPU is visible:
a valid call would then launch kernels on placeholder addresses."""

import ctypes
import math

import pytest
from hypothesis import HealthCheck, assume, given, settings
from hypothesis import strategies as st

import mla_latent_kv_10_amd as m

ROW_BYTES = {m.MLA_KV_BF16: 1152, m.MLA_KV_FP8_656: 656, m.MLA_KV_FP8_528: 528}
MAX_UNITS = 8192
MAX_SEQ_TOKENS = 1 << 23
STATIC_SCRATCH = 64 << 20
BASE = 1 << 30  # placeholder device addresses, 256-byte aligned and never dereferenced


@pytest.fixture(autouse=True)
def _no_gpu():
    # decided when a test runs, not at import: collecting this module (also in
    # a GPU run that deselects it) must not touch the HIP runtime
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: valid calls would launch kernels")


def n_row_groups(batch, s_q, h_q, sparse):
    """Row-group sequences of a call, by the header's split-policy rule."""
    R = h_q if sparse else s_q * h_q
    rg = 16 if R <= 16 else (64 if R <= 64 else 128)
    return batch * (s_q if sparse else 1) * math.ceil(R / rg)


@st.composite
def valid_calls(draw):
    fmt = draw(st.sampled_from(sorted(ROW_BYTES)))
    sparse = draw(st.booleans())
    batch = draw(st.integers(1, 300))
    s_q = draw(st.integers(1, 64))
    h_q = draw(st.integers(1, 256))
    assume(n_row_groups(batch, s_q, h_q, sparse) <= MAX_UNITS)
    a = m.MlaDecodeArgs()
    a.struct_size = ctypes.sizeof(m.MlaDecodeArgs)
    a.batch, a.s_q, a.h_q = batch, s_q, h_q
    ptrs = iter(BASE + 4096 * k for k in range(1, 32))
    a.q, a.kv, a.o, a.lse = next(ptrs), next(ptrs), next(ptrs), next(ptrs)
    a.row_bytes = ROW_BYTES[fmt]
    a.kv_format = fmt
    a.num_blocks = draw(st.integers(1, (1 << 32) // (64 * a.row_bytes)))
    a.block_size = 64
    if sparse:
        a.indices = next(ptrs)
        a.topk = draw(st.integers(1, min(MAX_SEQ_TOKENS, ((1 << 29) - 1) // (batch * s_q))))
        a.causal = 0
        a.block_table = a.cache_seqlens = 0
        a.max_blocks_per_seq = 1
    else:
        a.indices = 0
        a.topk = 0
        a.causal = draw(st.integers(0, 1))
        a.block_table, a.cache_seqlens = next(ptrs), next(ptrs)
        a.max_blocks_per_seq = draw(st.integers(1, MAX_SEQ_TOKENS // 64))
    a.softmax_scale = draw(st.floats(allow_nan=False, allow_infinity=False, width=32))
    a.tile_meta, a.split_offsets = next(ptrs), next(ptrs)
    a.num_parts = draw(st.integers(1, 65535))
    a.workspace = next(ptrs)
    need = ctypes.c_size_t(0)
    assert m.lib().mla_workspace_size(batch, s_q, h_q, a.num_parts, ctypes.byref(need)) == m.MLA_OK
    a.workspace_bytes = need.value + draw(st.integers(0, 4096))
    return a


def kind_workspace_bytes(batch, s_q, h_q, num_parts, sparse):
    """Split workspace of one kind of call, from the layout the header gives:
    S = Q + num_parts slots of RG x 512 fp16 partial rows, then (from the
    next 256-byte boundary) fp32 lse [S][RG] and fp32 scales [S][RG]."""
    R = h_q if sparse else s_q * h_q
    rg = 16 if R <= 16 else (64 if R <= 64 else 128)
    S = n_row_groups(batch, s_q, h_q, sparse) + num_parts
    return -(-(S * rg * 512 * 2) // 256) * 256 + 2 * S * rg * 4


def _call(fn, a):
    rc = fn(ctypes.byref(a), None)
    return rc, m.lib().mla_last_error().decode()


SETTINGS = settings(max_examples=2000, deadline=None, suppress_health_check=[HealthCheck.filter_too_much])


@SETTINGS
@given(valid_calls())
def test_documented_valid_calls_pass_validation(a):
    L = m.lib()
    for fn in (L.mla_decode_with_kvcache, L.mla_decode_splits, L.mla_combine):
        rc, msg = _call(fn, a)
        assert rc == m.MLA_ERR_HIP, (fn.__name__, rc, msg)
    # the size query covers both kinds of call the shape allows
    sizes = [kind_workspace_bytes(a.batch, a.s_q, a.h_q, a.num_parts, sp) for sp in (False, True)
             if n_row_groups(a.batch, a.s_q, a.h_q, sp) <= MAX_UNITS]
    need = ctypes.c_size_t(0)
    assert L.mla_workspace_size(a.batch, a.s_q, a.h_q, a.num_parts, ctypes.byref(need)) == m.MLA_OK
    assert need.value == max(sizes)
    # the entry point without a workspace: refused on the host when the call
    # needs more split workspace than its static scratch, else it reaches HIP
    rc, msg = _call(L.mla_decode_with_kvcache_static, a)
    over = kind_workspace_bytes(a.batch, a.s_q, a.h_q, a.num_parts, bool(a.indices)) > STATIC_SCRATCH
    assert rc == (m.MLA_ERR_UNSUPPORTED if over else m.MLA_ERR_HIP), (rc, msg)


def _mutations(a):
    """(label, field overrides, expected status, applies to the static entry)
    for one documented violation each, given the valid call a."""
    sparse = bool(a.indices)
    rb = a.row_bytes
    out = [
        ("struct_size", dict(struct_size=a.struct_size - 8), m.MLA_ERR_INVALID, True),
        ("batch < 1", dict(batch=0), m.MLA_ERR_INVALID, True),
        ("s_q < 1", dict(s_q=-1), m.MLA_ERR_INVALID, True),
        ("h_q < 1", dict(h_q=0), m.MLA_ERR_INVALID, True),
        ("num_parts 0", dict(num_parts=0), m.MLA_ERR_INVALID, True),
        ("num_parts 65536", dict(num_parts=65536), m.MLA_ERR_INVALID, True),
        ("q NULL", dict(q=0), m.MLA_ERR_INVALID, True),
        ("kv NULL", dict(kv=0), m.MLA_ERR_INVALID, True),
        ("o NULL", dict(o=0), m.MLA_ERR_INVALID, True),
        ("lse NULL", dict(lse=0), m.MLA_ERR_INVALID, True),
        ("q misaligned", dict(q=a.q + 8), m.MLA_ERR_INVALID, True),
        ("kv misaligned", dict(kv=a.kv + 4), m.MLA_ERR_INVALID, True),
        ("o misaligned", dict(o=a.o + 2), m.MLA_ERR_INVALID, True),
        ("lse misaligned", dict(lse=a.lse + 1), m.MLA_ERR_INVALID, True),
        ("block_size 32", dict(block_size=32), m.MLA_ERR_UNSUPPORTED, True),
        ("kv_format unknown", dict(kv_format=3), m.MLA_ERR_INVALID, True),
        ("row_bytes of another format", dict(row_bytes=[r for r in ROW_BYTES.values() if r != rb][0]),
         m.MLA_ERR_INVALID, True),
        ("num_blocks 0", dict(num_blocks=0), m.MLA_ERR_INVALID, True),
        ("cache above 4 GiB", dict(num_blocks=(1 << 32) // (64 * rb) + 1), m.MLA_ERR_UNSUPPORTED, True),
        ("softmax_scale NaN", dict(softmax_scale=float("nan")), m.MLA_ERR_INVALID, True),
        ("softmax_scale inf", dict(softmax_scale=float("inf")), m.MLA_ERR_INVALID, True),
        ("tile_meta NULL", dict(tile_meta=0), m.MLA_ERR_INVALID, True),
        ("split_offsets NULL", dict(split_offsets=0), m.MLA_ERR_INVALID, True),
        ("tile_meta misaligned", dict(tile_meta=a.tile_meta + 8), m.MLA_ERR_INVALID, True),
        ("split_offsets misaligned", dict(split_offsets=a.split_offsets + 2), m.MLA_ERR_INVALID, True),
        ("workspace NULL", dict(workspace=0), m.MLA_ERR_INVALID, False),
        ("workspace misaligned", dict(workspace=a.workspace + 128), m.MLA_ERR_INVALID, False),
        ("workspace too small", dict(workspace_bytes=16), m.MLA_ERR_WORKSPACE, False),
    ]
    per_unit = n_row_groups(1, a.s_q, a.h_q, sparse)
    out.append(("too many row-group sequences", dict(batch=MAX_UNITS // per_unit + 1), m.MLA_ERR_UNSUPPORTED, True))
    if sparse:
        out += [
            ("topk 0 with indices", dict(topk=0), m.MLA_ERR_INVALID, True),
            ("topk above 2^23", dict(topk=MAX_SEQ_TOKENS + 1), m.MLA_ERR_UNSUPPORTED, True),
            ("causal with indices", dict(causal=1), m.MLA_ERR_INVALID, True),
            ("indices misaligned", dict(indices=a.indices + 2), m.MLA_ERR_INVALID, True),
        ]
        topk_big = -(-(1 << 29) // (a.batch * a.s_q))
        if topk_big <= MAX_SEQ_TOKENS:
            out.append(("2^29 index entries", dict(topk=topk_big), m.MLA_ERR_UNSUPPORTED, True))
    else:
        out += [
            ("block_table NULL", dict(block_table=0), m.MLA_ERR_INVALID, True),
            ("cache_seqlens NULL", dict(cache_seqlens=0), m.MLA_ERR_INVALID, True),
            ("block_table misaligned", dict(block_table=a.block_table + 2), m.MLA_ERR_INVALID, True),
            ("cache_seqlens misaligned", dict(cache_seqlens=a.cache_seqlens + 1), m.MLA_ERR_INVALID, True),
            ("max_blocks_per_seq 0", dict(max_blocks_per_seq=0), m.MLA_ERR_INVALID, True),
            ("max_blocks_per_seq above 2^17", dict(max_blocks_per_seq=MAX_SEQ_TOKENS // 64 + 1),
             m.MLA_ERR_UNSUPPORTED, True),
            ("topk without indices", dict(topk=64), m.MLA_ERR_INVALID, True),
        ]
    return out


@SETTINGS
@given(valid_calls(), st.data())
def test_one_broken_field_gives_the_documented_status(a, data):
    L = m.lib()
    label, over, status, static_too = data.draw(st.sampled_from(_mutations(a)), label="mutation")
    b = m.MlaDecodeArgs.from_buffer_copy(a)
    for k, v in over.items():
        setattr(b, k, v)
    fns = [L.mla_decode_with_kvcache, L.mla_decode_splits, L.mla_combine]
    # the static entry tests its scratch capacity first: only calls that fit
    # it show the other statuses there
    fits = kind_workspace_bytes(a.batch, a.s_q, a.h_q, a.num_parts, bool(a.indices)) <= STATIC_SCRATCH
    if static_too and fits:
        fns.append(L.mla_decode_with_kvcache_static)
    for fn in fns:
        rc, msg = _call(fn, b)
        assert rc == status, (label, fn.__name__, rc, msg)
        assert msg, (label, fn.__name__)


@st.composite
def valid_metadata_calls(draw):
    sparse = draw(st.booleans())
    batch = draw(st.integers(1, 300))
    s_q = draw(st.integers(1, 64))
    h_q = draw(st.integers(1, 256))
    assume(n_row_groups(batch, s_q, h_q, sparse) <= MAX_UNITS)
    topk = draw(st.integers(1, MAX_SEQ_TOKENS)) if sparse else 0
    return dict(seqlens=0 if sparse else BASE + 4096, batch=batch, s_q=s_q, h_q=h_q, topk=topk,
                num_parts=draw(st.integers(1, 65535)), tile_meta=BASE + 8192, split_offsets=BASE + 12288)


def _metadata(c):
    L = m.lib()
    rc = L.mla_get_metadata(c["seqlens"], c["batch"], c["s_q"], c["h_q"], c["topk"], c["num_parts"],
                            c["tile_meta"], c["split_offsets"], None)
    return rc, L.mla_last_error().decode()


@SETTINGS
@given(valid_metadata_calls())
def test_documented_metadata_calls_pass_validation(c):
    rc, msg = _metadata(c)
    assert rc == m.MLA_ERR_HIP, (rc, msg)
    # the buffer sizes: num_parts rows of 8, and Q + 1 offsets for the larger
    # Q of the two kinds of call the shape allows
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    assert m.lib().mla_metadata_size(c["batch"], c["s_q"], c["h_q"], c["num_parts"], ctypes.byref(a),
                                     ctypes.byref(b)) == m.MLA_OK
    qs = [n_row_groups(c["batch"], c["s_q"], c["h_q"], sp) for sp in (False, True)]
    assert a.value == 8 * c["num_parts"]
    assert b.value == max(q for q in qs if q <= MAX_UNITS) + 1


@SETTINGS
@given(valid_metadata_calls(), st.data())
def test_metadata_with_one_broken_argument(c, data):
    per_unit = n_row_groups(1, c["s_q"], c["h_q"], c["topk"] > 0)
    cases = [
        ("batch < 1", dict(batch=0), m.MLA_ERR_INVALID),
        ("s_q < 1", dict(s_q=0), m.MLA_ERR_INVALID),
        ("h_q < 1", dict(h_q=-2), m.MLA_ERR_INVALID),
        ("topk < 0", dict(topk=-1), m.MLA_ERR_INVALID),
        ("topk above 2^23", dict(topk=MAX_SEQ_TOKENS + 1), m.MLA_ERR_UNSUPPORTED),
        ("num_parts 0", dict(num_parts=0), m.MLA_ERR_INVALID),
        ("num_parts 65536", dict(num_parts=65536), m.MLA_ERR_INVALID),
        ("tile_meta NULL", dict(tile_meta=0), m.MLA_ERR_INVALID),
        ("split_offsets NULL", dict(split_offsets=0), m.MLA_ERR_INVALID),
        ("tile_meta misaligned", dict(tile_meta=c["tile_meta"] + 4), m.MLA_ERR_INVALID),
        ("split_offsets misaligned", dict(split_offsets=c["split_offsets"] + 2), m.MLA_ERR_INVALID),
        ("too many row-group sequences", dict(batch=MAX_UNITS // per_unit + 1), m.MLA_ERR_UNSUPPORTED),
    ]
    if c["topk"] == 0:
        cases += [("cache_seqlens NULL", dict(seqlens=0), m.MLA_ERR_INVALID),
                  ("cache_seqlens misaligned", dict(seqlens=c["seqlens"] + 2), m.MLA_ERR_INVALID)]
    label, over, status = data.draw(st.sampled_from(cases), label="mutation")
    rc, msg = _metadata({**c, **over})
    assert rc == status and msg, (label, rc, msg)
