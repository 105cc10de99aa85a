"""Helpers shared by the GPU tests: move a workload to the GPU, run the HIP path
through the binding, evaluate the oracle on chosen query rows, compare."""

from __future__ import annotations

import math
import sys
from typing import Callable, Iterable, List, Optional, Tuple

import numpy as np
import torch

import mla_latent_kv_10_amd as mla
from oracle import attended_rows, decode_rows, mla_decode_ref

# Tolerances (the benchmark spec): bf16 o within 2e-2 max-abs; lse within 1e-3 of |lse|.
O_TOL = 2e-2
LSE_RTOL = 1e-3
# Where |lse_ref| < 1 the relative bound can fall below what fp32 arithmetic
# itself can promise; there the bound is the larger of the relative one and
# lse_fp32_floor (below). Everywhere else it is purely relative.
LSE_FLOOR_BELOW = 1.0

# bytes of NaN (0xFF) placed before and after the cache on the GPU
GUARD_BYTES = 64 * 1024

U32 = 2.0 ** -24  # unit roundoff of fp32


def gamma(n: float) -> float:
    """n u / (1 - n u): the classic bound on the relative error of n fp32 roundings."""
    return n * U32 / (1.0 - n * U32)


def lse_fp32_floor(q_norm: float, k_norm_max: float, n: int, scale: float) -> float:
    """Bound on |lse_fp32 - lse_exact| for one query row attending n keys.

    Each score is a 576-term dot product of bf16 values accumulated in fp32,
    then scaled: |s_hat - s| <= gamma(577) * scale * sum_d |q_d k_d|
    <= gamma(577) * scale * ||q|| * max_t ||k_t|| (Cauchy-Schwarz); lse moves
    by at most the largest score error. The sum of n exponentials (each within
    2 ulp) adds gamma(n + 3) relative to l, i.e. that much to ln l; the final
    m + log2(l) and the ln 2 product add a few ulp of |m| + |ln l|, with
    |m| <= scale * ||q|| * max ||k||.
    """
    smax = scale * q_norm * k_norm_max
    return gamma(577) * smax + gamma(n + 3) + 4 * U32 * (smax + math.log(max(n, 1)) + 1.0)


def lse_ok(got: float, ref: float, floor: float = 0.0) -> bool:
    tol = LSE_RTOL * abs(ref)
    if abs(ref) < LSE_FLOOR_BELOW:
        tol = max(tol, floor)
    return abs(got - ref) <= tol


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def guarded_copy(t: torch.Tensor, device="cuda:0", guard: int = GUARD_BYTES) -> torch.Tensor:
    """t on the GPU inside a larger buffer of NaN bytes: `guard` bytes of 0xFF
    before and after it, so a read one row (or a page) outside the cache sees
    NaN instead of another tensor's data. Returns the interior view."""
    n = t.numel() * t.element_size()
    big = torch.full((guard + n + guard,), 0xFF, dtype=torch.uint8, device=device)
    inner = big[guard:guard + n]
    inner.copy_(t.contiguous().view(torch.uint8).reshape(-1).to(device))
    return inner.view(t.dtype).view(t.shape)


def to_gpu(w, device="cuda:0", guard: bool = True):
    d = {
        "q": w.q.to(device),
        "kv": guarded_copy(w.kv, device) if guard else w.kv.to(device),
        "block_table": None if w.block_table is None else w.block_table.to(device),
        "cache_seqlens": w.cache_seqlens.to(device),
        "indices": None if w.indices is None else w.indices.to(device),
    }
    return d


def run_gpu(w, g=None, num_parts: Optional[int] = None, device="cuda:0"):
    """Metadata + decode on the GPU for workload w; returns (o, lse, tile_meta, split_offsets) on the GPU."""
    if g is None:
        g = to_gpu(w, device)
    tm, so = mla.get_mla_metadata(g["cache_seqlens"] if w.indices is None else None, w.s_q, w.h_q,
                                  topk=w.topk, num_parts=num_parts, batch=w.batch)
    o, lse = mla.mla_decode_with_kvcache(g["q"], g["kv"], g["block_table"], g["cache_seqlens"],
                                         448 if w.kv_format == "fp8_528" else 512, tm, so,
                                         softmax_scale=w.softmax_scale, causal=w.causal,
                                         is_fp8_kvcache=(w.kv_format != "bf16"), indices=g["indices"])
    return o, lse, tm, so


def _np_inputs(w):
    q = w.q.view(torch.int16).numpy().view(np.uint16)
    bt = None if w.block_table is None else w.block_table.numpy()
    idx = None if w.indices is None else w.indices.numpy()
    return q, bt, idx


def oracle(w, rows: Optional[Iterable[Tuple[int, int]]] = None):
    """The oracle on the chosen (b, i) rows (all by default).

    Rows are evaluated in chunks: one sequence (dense: the causal limit needs
    the sequence's own s_q) or a run of query positions of one sequence
    (sparse: indices name each position's rows, so a slice along s_q is the
    same call); each chunk calls the oracle on its slice of the inputs, so q
    is converted only where it is used. Rows not asked for stay NaN.
    """
    q, bt, idx = _np_inputs(w)
    kv = w.kv.numpy()
    seq = w.cache_seqlens.numpy()
    B, S = w.batch, w.s_q
    want = [(b, i) for b in range(B) for i in range(S)] if rows is None else list(rows)
    o = np.full((B, S, w.h_q, 448 if w.kv_format == "fp8_528" else 512), np.nan)
    lse = np.full((B, S, w.h_q), np.nan)
    by_b = {}
    for b, i in want:
        by_b.setdefault(b, []).append(i)
    for b, its in sorted(by_b.items()):
        its = sorted(set(its))
        step = S if idx is None else 16
        for k in range(0, len(its), step):
            part = its[k:k + step]
            i0, i1 = (0, S) if idx is None else (part[0], part[-1] + 1)
            oo, ll = mla_decode_ref(q[b:b + 1, i0:i1], kv, w.kv_format,
                                    block_table=None if bt is None else bt[b:b + 1],
                                    cache_seqlens=seq[b:b + 1], softmax_scale=w.softmax_scale, causal=w.causal,
                                    indices=None if idx is None else idx[b:b + 1, i0:i1],
                                    rows=[(0, i - i0) for i in part])
            for i in part:
                o[b, i] = oo[0, i - i0]
                lse[b, i] = ll[0, i - i0]
    return o, lse


def workload_floor_fn(w) -> Callable[[int, int], np.ndarray]:
    """(b, i) -> per-head lse_fp32_floor for workload w (computed on demand)."""
    q, bt, idx = _np_inputs(w)
    kv = w.kv.numpy()
    flat = kv.reshape(-1, kv.shape[-1])
    seq = w.cache_seqlens.numpy()

    def fn(b, i):
        r = attended_rows(b, i, s_q=w.s_q, num_rows=flat.shape[0], block_table=bt, cache_seqlens=seq,
                          causal=w.causal, indices=idx)
        K = decode_rows(flat[r], w.kv_format)
        qb = (q[b, i].astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        kmax = float(np.sqrt((K ** 2).sum(axis=1)).max()) if len(r) else 0.0
        return np.array([lse_fp32_floor(float(np.linalg.norm(qb[h])), kmax, len(r), w.softmax_scale)
                         for h in range(w.h_q)])

    return fn


def compare(o_gpu, lse_gpu, o_ref, lse_ref, rows: Optional[List[Tuple[int, int]]] = None, label="",
            floor_fn: Optional[Callable[[int, int], np.ndarray]] = None):
    """o within O_TOL max-abs; lse within LSE_RTOL * |lse_ref|, or (only where
    |lse_ref| < 1) within the fp32 floor that floor_fn(b, i) gives per head;
    rows with no attended token must be exactly o = 0, lse = -inf."""
    og = o_gpu.float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.cpu().numpy().astype(np.float64)
    if rows is None:
        B, S = og.shape[:2]
        rows = [(b, i) for b in range(B) for i in range(S)]
    worst_o = 0.0
    worst_l = 0.0
    for b, i in rows:
        ro, rl = o_ref[b, i], lse_ref[b, i]
        go, gl = og[b, i], lg[b, i]
        assert np.all(np.isfinite(go)), f"{label} non-finite o at {(b, i)}"
        empty = ~np.isfinite(rl)
        assert np.array_equal(np.isinf(gl) & (gl < 0), empty), f"{label} -inf lse mismatch at {(b, i)}"
        if np.any(empty):
            assert np.all(go[empty] == 0), f"{label} empty rows must be zero at {(b, i)}"
        ne = ~empty
        if np.any(ne):
            eo = float(np.max(np.abs(go[ne] - ro[ne])))
            worst_o = max(worst_o, eo)
            err = np.abs(gl - rl)
            rel = np.where(ne, err / np.maximum(np.abs(rl), 1e-300), 0.0)
            small = ne & (np.abs(rl) < LSE_FLOOR_BELOW) & (err > LSE_RTOL * np.abs(rl))
            if np.any(small):
                floor = floor_fn(b, i) if floor_fn is not None else np.zeros_like(rl)
                for h in np.nonzero(small)[0]:
                    assert lse_ok(gl[h], rl[h], floor[h]), \
                        f"{label}: lse {gl[h]} vs {rl[h]} at {(b, i, int(h))}, fp32 floor {floor[h]:.3e}"
                    rel[h] = 0.0
            worst_l = max(worst_l, float(np.max(rel[ne])))
    say(f"  {label}: max|do| = {worst_o:.3e} (tol {O_TOL}), max rel dlse = {worst_l:.3e} (tol {LSE_RTOL})")
    assert worst_o <= O_TOL, f"{label}: o error {worst_o}"
    assert worst_l <= LSE_RTOL, f"{label}: lse error {worst_l}"
    return worst_o, worst_l
