"""MI355X (gfx950) MLA decode over a paged latent KV cache.

Python binding of the C ABI in include/mla.h. This module only marshals
arguments: every step of the decode runs in the HIP library
libmla_mi355x.so, which is built in-tree (``python -m
mla_latent_kv_10_amd.build``). There is no fallback path: if the library or
a GPU is missing, calls raise.

Call shape (as in the FlashMLA usage guide page, §"怎么用起来"):

    tile_meta, split_offsets = get_mla_metadata(cache_seqlens, s_q, h_q, topk)
    o, lse = mla_decode_with_kvcache(q, kv, block_table, cache_seqlens, 512,
                                     tile_meta, split_offsets, softmax_scale,
                                     causal, is_fp8_kvcache, indices)
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_mi355x.so")
# the race-check build: the split kernel waits for each tile's loads right
# after issuing them (same entry points; used only by the LDS race check)
DRAIN_LIB_PATH = os.path.join(HERE, "libmla_mi355x_drain.so")

MLA_OK = 0
MLA_ERR_INVALID = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE = -3
MLA_ERR_HIP = -4
MLA_KV_BF16 = 0
MLA_KV_FP8_656 = 1
MLA_KV_FP8_528 = 2
ROW_BYTES = {MLA_KV_BF16: 1152, MLA_KV_FP8_656: 656, MLA_KV_FP8_528: 528}
# (key / query dims, value / output dims) per cache format
DIMS = {MLA_KV_BF16: (576, 512), MLA_KV_FP8_656: (576, 512), MLA_KV_FP8_528: (512, 448)}


class MlaDecodeArgs(ctypes.Structure):
    """Mirror of ``mla_decode_args`` (include/mla.h), same field order."""

    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("s_q", ctypes.c_int32),
        ("h_q", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("kv", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("row_bytes", ctypes.c_int32),
        ("kv_format", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("cache_seqlens", ctypes.c_void_p),
        ("indices", ctypes.c_void_p),
        ("topk", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("tile_meta", ctypes.c_void_p),
        ("split_offsets", ctypes.c_void_p),
        ("num_parts", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
    ]


EXPORTS = (
    "mla_last_error",
    "mla_default_num_parts",
    "mla_metadata_size",
    "mla_workspace_size",
    "mla_get_metadata",
    "mla_decode_with_kvcache",
    "mla_decode_splits",
    "mla_combine",
    "mla_decode_with_kvcache_static",
    "mla_quantize_fp8_append",
    "mla_absorb_q",
    "mla_unabsorb_o",
    "mla_probe_mfma_bf16",
    "mla_probe_hbm_read",
)

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmla_mi355x.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


_drain_lib = None


def drain_lib() -> ctypes.CDLL:
    """Load the race-check build libmla_mi355x_drain.so (same entry points)."""
    global _drain_lib
    if _drain_lib is None:
        _drain_lib = _load(DRAIN_LIB_PATH)
    return _drain_lib


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing; build it with `python -m mla_latent_kv_10_amd.build`")
    # One HIP runtime per process. torch, when installed, ships its own
    # libamdhip64 under the same soname; with torch loaded first this library
    # binds to that copy. Loaded first, it would bring in the system's copy,
    # and torch's own would then find no devices.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(path)
    L.mla_last_error.restype = ctypes.c_char_p
    L.mla_last_error.argtypes = []
    L.mla_default_num_parts.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    L.mla_metadata_size.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_int64)] * 2
    L.mla_workspace_size.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_size_t)]
    L.mla_get_metadata.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.mla_decode_with_kvcache.argtypes = [ctypes.POINTER(MlaDecodeArgs), ctypes.c_void_p]
    L.mla_decode_splits.argtypes = [ctypes.POINTER(MlaDecodeArgs), ctypes.c_void_p]
    L.mla_combine.argtypes = [ctypes.POINTER(MlaDecodeArgs), ctypes.c_void_p]
    L.mla_decode_with_kvcache_static.argtypes = [ctypes.POINTER(MlaDecodeArgs), ctypes.c_void_p]
    L.mla_quantize_fp8_append.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_int64, ctypes.c_void_p]
    L.mla_absorb_q.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                               ctypes.c_void_p, ctypes.c_void_p]
    L.mla_unabsorb_o.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p]
    L.mla_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    L.mla_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    for name in EXPORTS:
        getattr(L, name).restype = ctypes.c_char_p if name == "mla_last_error" else ctypes.c_int
    return L


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"mla status {status}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != MLA_OK:
        raise MlaError(status, lib().mla_last_error().decode())


# ---------------------------------------------------------------- sizes

def default_num_parts(device: int = 0) -> int:
    n = ctypes.c_int(0)
    check(lib().mla_default_num_parts(device, ctypes.byref(n)))
    return n.value


def metadata_size(batch: int, s_q: int, h_q: int, num_parts: int) -> Tuple[int, int]:
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    check(lib().mla_metadata_size(batch, s_q, h_q, num_parts, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def workspace_size(batch: int, s_q: int, h_q: int, num_parts: int) -> int:
    n = ctypes.c_size_t(0)
    check(lib().mla_workspace_size(batch, s_q, h_q, num_parts, ctypes.byref(n)))
    return n.value


# ---------------------------------------------------------------- torch-facing calls

def _torch():
    import torch

    return torch


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _require_gpu(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _expect(t, label: str, dtype, shape) -> None:
    """t must have this dtype and shape (None in shape: any size there)."""
    if t is None:
        raise ValueError(f"{label} is required")
    if t.dtype != dtype:
        raise ValueError(f"{label} must be {dtype} (got {t.dtype})")
    if t.dim() != len(shape) or any(w is not None and g != w for g, w in zip(t.shape, shape)):
        want = ", ".join("*" if w is None else str(w) for w in shape)
        raise ValueError(f"{label} must have shape [{want}] (got {list(t.shape)})")


def cache_format(kv, is_fp8_kvcache: bool) -> int:
    """The cache's row format: bf16 (576 bf16 values, or 1152 bytes), FP8 with
    656-byte rows, or FP8 with 528-byte rows (both uint8 [num_blocks, 64, row])."""
    torch = _torch()
    if is_fp8_kvcache:
        if kv is not None and kv.dtype == torch.uint8 and kv.dim() == 3 and kv.shape[2] == 528:
            _expect(kv, "kv (FP8 cache, 528-byte rows)", torch.uint8, (None, 64, 528))
            return MLA_KV_FP8_528
        _expect(kv, "kv (FP8 cache: 656- or 528-byte rows)", torch.uint8, (None, 64, 656))
        return MLA_KV_FP8_656
    if kv is not None and kv.dtype == torch.bfloat16:
        _expect(kv, "kv (bf16 cache)", torch.bfloat16, (None, 64, 576))
    else:
        _expect(kv, "kv (bf16 cache as bytes)", torch.uint8, (None, 64, 1152))
    return MLA_KV_BF16


def get_mla_metadata(cache_seqlens, s_q: int, h_q: int, topk: int = 0, num_parts: Optional[int] = None,
                     batch: Optional[int] = None):
    """Split schedule for one decode step; returns (tile_meta, split_offsets) int32 GPU tensors."""
    torch = _torch()
    if cache_seqlens is not None:
        _require_gpu(cache_seqlens)
        if cache_seqlens.dtype != torch.int32:
            raise ValueError("cache_seqlens must be int32")
        batch = cache_seqlens.numel()
        device = cache_seqlens.device
    else:
        device = torch.device("cuda", torch.cuda.current_device())
    if num_parts is None:
        num_parts = default_num_parts(device.index or 0)
    n_meta, n_off = metadata_size(batch, s_q, h_q, num_parts)
    tile_meta = torch.empty((num_parts, 8), dtype=torch.int32, device=device)
    split_offsets = torch.empty((n_off,), dtype=torch.int32, device=device)
    check(lib().mla_get_metadata(_ptr(cache_seqlens), batch, s_q, h_q, topk, num_parts, tile_meta.data_ptr(),
                                 split_offsets.data_ptr(), _stream_handle(device)))
    # the call shape the schedule was built for; the decode compares it
    tile_meta.mla_call_shape = (batch, s_q, h_q, topk)
    return tile_meta, split_offsets


def make_args(q, kv, block_table, cache_seqlens, tile_meta, split_offsets, softmax_scale, causal, is_fp8_kvcache,
              indices, workspace, o, lse) -> MlaDecodeArgs:
    """Argument block for the decode entry points, after checking every tensor.

    q bf16 [B, s_q, h_q, 576]; kv [num_blocks, 64, 576] bf16 or [num_blocks,
    64, 1152] uint8 (bf16 cache), [num_blocks, 64, 656] uint8 (FP8 cache);
    with an FP8 cache of 528-byte rows q has 512 dims and o 448;
    dense: block_table int32 [B, max_blocks_per_seq] and cache_seqlens int32
    [B]; sparse: indices int32 [B, s_q, topk]; tile_meta int32 [num_parts, 8]
    and split_offsets int32 [Q + 1] from get_mla_metadata for this (B, s_q,
    h_q, topk); workspace uint8 with at least workspace_size(...) bytes; o bf16
    [B, s_q, h_q, 512]; lse fp32 [B, s_q, h_q]. All contiguous, on q's device.
    Raises ValueError naming the first tensor that does not fit.
    """
    torch = _torch()
    fmt = cache_format(kv, is_fp8_kvcache)
    d_qk, d_v = DIMS[fmt]
    _expect(q, "q", torch.bfloat16, (None, None, None, d_qk))
    batch, s_q, h_q, _ = q.shape
    if indices is None:
        _expect(block_table, "block_table", torch.int32, (batch, None))
        _expect(cache_seqlens, "cache_seqlens", torch.int32, (batch,))
        topk = 0
    else:
        _expect(indices, "indices", torch.int32, (batch, s_q, None))
        topk = indices.shape[2]
    _expect(tile_meta, "tile_meta", torch.int32, (None, 8))
    num_parts = tile_meta.shape[0]
    _, n_off = metadata_size(batch, s_q, h_q, num_parts)
    _expect(split_offsets, "split_offsets", torch.int32, (n_off,))
    built = getattr(tile_meta, "mla_call_shape", None)
    if built is not None and tuple(built) != (batch, s_q, h_q, topk):
        raise ValueError(f"metadata was built for (batch, s_q, h_q, topk) = {tuple(built)}, "
                         f"this call is {(batch, s_q, h_q, topk)}: call get_mla_metadata again")
    _expect(workspace, "workspace", torch.uint8, (None,))
    _expect(o, "o", torch.bfloat16, (batch, s_q, h_q, d_v))
    _expect(lse, "lse", torch.float32, (batch, s_q, h_q))
    tensors = [q, kv, tile_meta, split_offsets, workspace, o, lse]
    tensors += [block_table, cache_seqlens] if indices is None else [indices]
    _require_gpu(*tensors)
    if any(t.device != q.device for t in tensors):
        raise ValueError("all tensors must be on q's device")
    a = MlaDecodeArgs()
    a.struct_size = ctypes.sizeof(MlaDecodeArgs)
    a.batch, a.s_q, a.h_q = batch, s_q, h_q
    a.q, a.kv = q.data_ptr(), kv.data_ptr()
    a.num_blocks = kv.shape[0]
    a.block_size = kv.shape[1]
    a.row_bytes = kv[0, 0].numel() * kv.element_size()
    a.kv_format = fmt
    a.block_table = _ptr(block_table) if indices is None else 0
    a.max_blocks_per_seq = block_table.shape[1] if indices is None else 0
    a.cache_seqlens = _ptr(cache_seqlens) if indices is None else 0
    a.indices = _ptr(indices)
    a.topk = topk
    a.softmax_scale = float(softmax_scale)
    a.causal = 1 if causal else 0
    a.tile_meta, a.split_offsets = tile_meta.data_ptr(), split_offsets.data_ptr()
    a.num_parts = num_parts
    a.workspace = workspace.data_ptr()
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    a.o, a.lse = o.data_ptr(), lse.data_ptr()
    return a


def mla_decode_with_kvcache(q, kv, block_table, cache_seqlens, head_dim_v: int, tile_meta, split_offsets,
                            softmax_scale: Optional[float] = None, causal: bool = False,
                            is_fp8_kvcache: bool = False, indices=None, workspace=None, out=None):
    """Decode attention; returns (o bf16 [B, s_q, h_q, d_v], lse fp32 [B, s_q, h_q]).

    d_v (head_dim_v) is 512, or 448 for an FP8 cache of 528-byte rows (whose q has 512 dims).
    """
    torch = _torch()
    fmt = cache_format(kv, is_fp8_kvcache)
    d_qk, d_v = DIMS[fmt]
    if head_dim_v != d_v:
        raise ValueError(f"head_dim_v must be {d_v} for this cache format")
    _expect(q, "q", torch.bfloat16, (None, None, None, d_qk))
    _expect(tile_meta, "tile_meta", torch.int32, (None, 8))
    batch, s_q, h_q, _ = q.shape
    if softmax_scale is None:
        softmax_scale = 576 ** -0.5
    num_parts = tile_meta.shape[0]
    if workspace is None:
        workspace = torch.empty((workspace_size(batch, s_q, h_q, num_parts),), dtype=torch.uint8, device=q.device)
    if out is None:
        o = torch.empty((batch, s_q, h_q, d_v), dtype=torch.bfloat16, device=q.device)
        lse = torch.empty((batch, s_q, h_q), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
    a = make_args(q, kv, block_table, cache_seqlens, tile_meta, split_offsets, softmax_scale, causal,
                  is_fp8_kvcache, indices, workspace, o, lse)
    check(lib().mla_decode_with_kvcache(ctypes.byref(a), _stream_handle(q.device)))
    return o, lse


def mla_decode_splits(args: MlaDecodeArgs, stream: int) -> None:
    """Run only the split kernel for a prepared argument block (mla_combine must follow)."""
    check(lib().mla_decode_splits(ctypes.byref(args), stream))


def mla_decode_static(args: MlaDecodeArgs, stream: int) -> None:
    """mla_decode_with_kvcache on the library's static scratch (allocates nothing; workspace fields ignored)."""
    check(lib().mla_decode_with_kvcache_static(ctypes.byref(args), stream))


def mla_combine(args: MlaDecodeArgs, stream: int) -> None:
    """Run only the split merge for a prepared argument block."""
    check(lib().mla_combine(ctypes.byref(args), stream))


def quantize_fp8_append(src, slots, kv) -> None:
    """Quantise bf16 rows src [n, 576] into the FP8 cache kv [num_blocks, 64, 656] (uint8) at rows slots [n]."""
    torch = _torch()
    _require_gpu(src, slots, kv)
    if src.dtype != torch.bfloat16 or src.dim() != 2 or src.shape[1] != 576:
        raise ValueError("src must be bfloat16 [n, 576]")
    if slots.dtype != torch.int32 or slots.shape != (src.shape[0],):
        raise ValueError("slots must be int32 [n]")
    if kv.dtype != torch.uint8 or kv.dim() != 3 or tuple(kv.shape[1:]) != (64, 656):
        raise ValueError("kv must be uint8 [num_blocks, 64, 656]")
    check(lib().mla_quantize_fp8_append(src.data_ptr(), slots.data_ptr(), src.shape[0], kv.data_ptr(), kv.shape[0],
                                        _stream_handle(src.device)))


def absorb_q(q_nope, q_rope, w_uk_t, out=None):
    """Absorbed queries [T, H, 576] from q_nope [T, H, 128], q_rope [T, H, 64] and w_uk_t [H, 512, 128] (bf16)."""
    torch = _torch()
    _require_gpu(q_nope, q_rope, w_uk_t, out)
    T, H, dn = q_nope.shape
    for t, shape, label in ((q_nope, (T, H, 128), "q_nope"), (q_rope, (T, H, 64), "q_rope"),
                            (w_uk_t, (H, 512, 128), "w_uk_t")):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != shape:
            raise ValueError(f"{label} must be bfloat16 {list(shape)}")
    if out is None:
        out = torch.empty((T, H, 576), dtype=torch.bfloat16, device=q_nope.device)
    elif out.dtype != torch.bfloat16 or out.numel() != T * H * 576:
        raise ValueError("out must be bfloat16 with T * H * 576 elements")
    check(lib().mla_absorb_q(q_nope.data_ptr(), q_rope.data_ptr(), w_uk_t.data_ptr(), T, H, out.data_ptr(),
                             _stream_handle(q_nope.device)))
    return out


def unabsorb_o(o_latent, w_uv):
    """Per-head outputs [T, H, 128] = W^UV_h o_latent[t, h] from o_latent [T, H, 512] and w_uv [H, 128, 512] (bf16)."""
    torch = _torch()
    _require_gpu(o_latent, w_uv)
    T, H, dc = o_latent.shape
    if o_latent.dtype != torch.bfloat16 or dc != 512:
        raise ValueError("o_latent must be bfloat16 [T, H, 512]")
    if w_uv.dtype != torch.bfloat16 or tuple(w_uv.shape) != (H, 128, 512):
        raise ValueError("w_uv must be bfloat16 [H, 128, 512]")
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=o_latent.device)
    check(lib().mla_unabsorb_o(o_latent.data_ptr(), w_uv.data_ptr(), T, H, out.data_ptr(),
                               _stream_handle(o_latent.device)))
    return out



# ---------------------------------------------------------------- measurement aids


def probe_mfma_bf16(iters: int, blocks: int, value: float, sink) -> None:
    """Enqueue the MFMA loop (blocks x 4 waves x iters x 4 MFMAs of 32x32x16 bf16) on the current stream.

    sink: float32 [blocks * 256] on the GPU, receives 1024 * iters * bf16(value)^2 per thread.
    """
    torch = _torch()
    _require_gpu(sink)
    if sink.dtype != torch.float32 or sink.numel() < blocks * 256:
        raise ValueError("sink must be float32 with at least blocks * 256 elements")
    check(lib().mla_probe_mfma_bf16(iters, blocks, value, sink.data_ptr(), _stream_handle(sink.device)))


def probe_hbm_read(src, blocks: int, sink) -> None:
    """Enqueue one non-temporal read of every byte of src (a multiple of 16 bytes) on the current stream.

    sink: int32 [blocks * 256] on the GPU, receives per thread the sum mod 2^32 of the words it read.
    """
    torch = _torch()
    _require_gpu(src, sink)
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    if sink.dtype != torch.int32 or sink.numel() < blocks * 256:
        raise ValueError("sink must be int32 with at least blocks * 256 elements")
    nbytes = src.numel() * src.element_size()
    check(lib().mla_probe_hbm_read(src.data_ptr(), nbytes, blocks, sink.data_ptr(), _stream_handle(src.device)))
