"""mla_combine through the C ABI on hand-made partials vs the oracle's split merge."""

import ctypes

import numpy as np
import pytest
import torch

import mla_latent_kv_10_amd as mla
from oracle import lse_merge

from tests.gpu_helpers import O_TOL, U32, gamma, lse_ok, say

pytestmark = pytest.mark.gpu


def _slot_layout(part_o):
    """Logical partials [S][RG][512] -> the documented workspace layout
    (RG = 16 row-major; RG = 128 or 64 blocked: 4-value group
    ((w*16+dd)*4+g)*64+lane holds row 32w+(lane&31), dims 32dd+8g+4(lane>>5)+0..3)."""
    S, RG, _ = part_o.shape
    if RG == 16:
        return np.ascontiguousarray(part_o)
    out = np.empty((S, RG // 32, 16, 4, 64, 4), dtype=part_o.dtype)
    for w in range(RG // 32):
        for lane in range(64):
            r = 32 * w + (lane & 31)
            h = lane >> 5
            for dd in range(16):
                for g in range(4):
                    d0 = 32 * dd + 8 * g + 4 * h
                    out[:, w, dd, g, lane, :] = part_o[:, r, d0:d0 + 4]
    return out.reshape(S, RG, 512)


@pytest.mark.parametrize("B,h_q,s_q,P,max_splits", [(3, 128, 1, 8, 5), (3, 64, 1, 64, 5), (3, 16, 2, 8, 5),
                                                   (3, 20, 1, 8, 5), (3, 100, 2, 8, 5), (10, 128, 1, 200, 40),
                                                   (10, 16, 1, 200, 40), (6, 64, 2, 240, 40), (8, 128, 1, 32, 9),
                                                   (8, 64, 2, 48, 7), (48, 128, 1, 48, 3), (24, 64, 2, 48, 3)])
def test_combine_matches_oracle_merge(B, h_q, s_q, P, max_splits):
    """Split counts 0..max_splits-1: every chunk size of the merge (2, 4, 8, 16
    splits in flight), sequences spanning several chunks, and both thread
    mappings of the blocked layouts (num_parts <= sequences selects the
    wide one: 8 groups per thread, chunks of at most 4 splits). Workspace
    bytes past the used slots hold NaN, and the last sequence's split count
    is not a multiple of its chunk width, so a load slot past a chunk's last
    split that read beyond the chunk would turn its zero weight into NaN."""
    say(f"combine h_q={h_q} s_q={s_q} parts={P} splits<{max_splits}")
    dev = "cuda:0"
    # a dense call: all s_q * h_q rows of a sequence in one row space
    R = s_q * h_q
    RG = 16 if R <= 16 else (64 if R <= 64 else 128)
    n_hb = -(-R // RG)
    n_rg = n_hb
    Q = B * n_rg
    rng = np.random.default_rng(h_q + s_q)
    n_splits = rng.integers(0, max_splits, Q)
    n_splits[0] = 3
    if Q > 2:
        n_splits[1] = 1
        n_splits[2] = 0
    if P <= Q and Q > 3:
        n_splits[3] = 9   # the wide mapping: one sequence over three chunks
    if Q > 4:
        n_splits[Q - 1] = 3   # chunk of 4 with one slot past the last split
    offs = np.zeros(Q + 1, dtype=np.int32)
    offs[1:] = np.cumsum(n_splits)
    S = Q + P
    assert offs[-1] <= S, (offs[-1], S)
    # stored rows: fp16 values h with a power-of-two scale c per (slot, row), of
    # magnitudes far apart; the partial the merge sees is c * h (exact in fp64)
    part_h = rng.standard_normal((S, RG, 512)).astype(np.float16)
    part_c = np.exp2(rng.integers(-30, 30, (S, RG))).astype(np.float32)
    part_c[0, :3] = 1.0
    part_o = part_h.astype(np.float64) * part_c[:, :, None].astype(np.float64)
    part_lse = (rng.standard_normal((S, RG)) * 3).astype(np.float32)
    part_lse[offs[0] + 1, :5] = -np.inf                     # an empty split
    o_bytes = ((S * RG * 512 * 2 + 255) // 256) * 256
    # only the slots the split offsets name are written; every other byte is
    # 0xFF (NaN as fp16 and as fp32)
    U = int(offs[-1])
    ws_bytes = mla.workspace_size(B, s_q, h_q, P)
    assert ws_bytes >= o_bytes + 2 * S * RG * 4
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device=dev)
    ws[:U * RG * 512 * 2] = torch.from_numpy(_slot_layout(part_h)[:U].view(np.uint8).reshape(-1)).to(dev)
    ws[o_bytes:o_bytes + U * RG * 4] = torch.from_numpy(part_lse[:U].view(np.uint8).reshape(-1)).to(dev)
    ws[o_bytes + S * RG * 4:o_bytes + S * RG * 4 + U * RG * 4] = torch.from_numpy(
        part_c[:U].view(np.uint8).reshape(-1)).to(dev)
    o = torch.full((B, s_q, h_q, 512), 7.0, dtype=torch.bfloat16, device=dev)   # sentinel
    lse = torch.full((B, s_q, h_q), 7.0, dtype=torch.float32, device=dev)
    q = torch.zeros((B, s_q, h_q, 576), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((1, 64, 1152), dtype=torch.uint8, device=dev)
    bt = torch.zeros((B, 1), dtype=torch.int32, device=dev)
    seq = torch.zeros((B,), dtype=torch.int32, device=dev)
    tm = torch.zeros((P, 8), dtype=torch.int32, device=dev)
    # the split-offset buffer has the size the size query gives (it covers a
    # sparse call of this shape too); the merge reads the first Q + 1
    _, n_off = mla.metadata_size(B, s_q, h_q, P)
    so_full = np.zeros(n_off, dtype=np.int32)
    so_full[:Q + 1] = offs
    so = torch.from_numpy(so_full).to(dev)
    a = mla.make_args(q, kv, bt, seq, tm, so, 0.1, False, False, None, ws, o, lse)
    mla.mla_combine(a, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    og = o.float().cpu().numpy()
    lg = lse.cpu().numpy()
    for qq in range(Q):
        b, hb = divmod(qq, n_rg)
        n = n_splits[qq]
        for r in range(RG):
            f = hb * RG + r          # row of the row space: position f // h_q, head f % h_q
            if f >= R:
                continue
            i, h = divmod(f, h_q)
            if n == 1:
                assert np.all(og[b, i, h] == 7.0) and lg[b, i, h] == 7.0   # left for the split kernel
                continue
            if n == 0:
                assert np.all(og[b, i, h] == 0) and lg[b, i, h] == -np.inf
                continue
            sl = slice(offs[qq], offs[qq + 1])
            ro, rl = lse_merge(part_o[sl, r], part_lse[sl, r].astype(np.float64))
            # relative to the row's magnitude (the scales span 2^-30 .. 2^29)
            assert np.max(np.abs(og[b, i, h] - ro)) <= O_TOL * max(1.0, np.max(np.abs(ro)))
            # fp32 merge: m + ln(sum_k e^{lse_k - m}); each exponent argument is
            # rounded twice (difference, base-2 scaling), each exponential and the
            # log are within 2 ulp, and the n-term sum adds gamma(n)
            lk = part_lse[sl, r].astype(np.float64)
            floor = gamma(n + 4) + 8 * U32 * (1.0 + 2.0 * float(np.max(np.abs(lk[np.isfinite(lk)]), initial=0.0)))
            assert lse_ok(lg[b, i, h], rl, floor), (qq, r, lg[b, i, h], rl, floor)
