"""Pins for the oracle's 528-byte row (CPU only): the UE8M0 scale values, the
row decode, the writer, and attention with 512-dim keys and 448-dim values.

Each check compares the oracle against something fixed outside it: a library
routine (math.ldexp, torch's e4m3 cast, torch's attention), a hand-worked
row, brute force over the scale exponent, or a closed form."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import E4M3FN_VALUES, attend, decode_rows, mla_decode_ref, quantize_rows_528, ue8m0_values
from workload import make_workload, quantize_fp8_528

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = float(np.float32(512 ** -0.5))


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_ue8m0_values_match_ldexp_for_every_byte():
    e = np.arange(256)
    v = ue8m0_values(e)
    for k in range(255):
        assert float(v[k]) == math.ldexp(1.0, k - 127), k
    assert math.isnan(float(v[255]))


def _golden_row():
    g = _load("fp8_row_528.json")
    row = np.zeros(528, dtype=np.uint8)
    for j, blk in enumerate(g["blocks"]):
        row[32 * j:32 * (j + 1)] = int(blk["code"], 16)
        row[512 + j] = blk["e"]
    return row, [b["value"] for b in g["blocks"]]


def test_528_row_golden():
    row, want = _golden_row()
    vals = decode_rows(row[None, :], "fp8_528")[0]
    assert vals.shape == (512,)
    for j, v in enumerate(want):
        blk = vals[32 * j:32 * (j + 1)]
        assert np.all(blk == v) and np.all(np.signbit(blk) == (math.copysign(1, v) < 0)), (j, blk[:2], v)


def test_528_writer_golden():
    for case in _load("fp8_quantize_row_528.json")["cases"]:
        x = np.zeros(512, dtype=np.float32)
        x[:len(case["block"])] = case["block"]
        out = quantize_rows_528(_bits(x[None, :]))[0]
        assert out[512] == case["e"], case["worked"]
        assert [int(c) for c in out[:len(case["codes"])]] == [int(c, 16) for c in case["codes"]], case["worked"]
        assert np.all(out[513:528] == 127) and np.all(out[len(case["codes"]):32] == 0)


def test_528_scale_is_the_smallest_power_of_two_covering_amax():
    """Brute force over k: 448 * 2^(k - 1) < amax <= 448 * 2^k."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((300, 512)) * np.exp(rng.uniform(-30, 30, (300, 16))).repeat(32, 1)).astype(np.float32)
    x[0, :32] = 448.0 * 2.0 ** -5        # amax exactly 448 * 2^k
    x[1, 32:64] = np.float32(448.0 * 2.0 ** 3) * np.float32(1 + 2 ** -7)   # just above
    x[2, 64:96] = 0.0
    b = _bits(x)
    xb = (b.astype(np.uint32) << 16).view(np.float32).reshape(300, 16, 32)
    out = quantize_rows_528(b)
    for r in range(300):
        for j in range(16):
            amax = float(np.abs(xb[r, j]).max())
            e = int(out[r, 512 + j])
            if amax == 0:
                assert e == 127
                continue
            k = next(k for k in range(-140, 140) if 448.0 * 2.0 ** k >= amax)
            assert e == k + 127, (r, j, amax, e)


def test_528_codes_match_torch_e4m3_cast():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((200, 512)) * 3).astype(np.float32)
    b = _bits(x)
    out = quantize_rows_528(b)
    xb = torch.from_numpy((b.astype(np.uint32) << 16).view(np.float32)).to(torch.float64).reshape(200, 16, 32)
    k = torch.from_numpy(out[:, 512:].astype(np.int64) - 127)
    y = torch.ldexp(xb, -k.unsqueeze(2)).to(torch.float32)
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(200, 512).numpy()
    assert np.array_equal(out[:, :512], ref)


def test_528_round_trip_bound_and_generator_agreement():
    """Writer then decode: e4m3 keeps 3 mantissa bits (half-ulp 2^-4 relative
    for normals, 2^-10 of the scale for subnormals) and the power-of-two scale
    adds no rounding. The input generator's torch writer gives the same bytes."""
    g = torch.Generator().manual_seed(6)
    x = torch.randn(400, 512, generator=g) * torch.exp(2 * torch.randn(400, 16, generator=g)).repeat_interleave(32, 1)
    xb = x.to(torch.bfloat16)
    rows = quantize_rows_528(xb.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(rows, quantize_fp8_528(xb.float()).numpy())
    dec = decode_rows(rows, "fp8_528")
    xv = xb.to(torch.float64).numpy()
    scale = np.repeat(ue8m0_values(rows[:, 512:]).astype(np.float64), 32, axis=1)
    assert np.all(np.abs(dec - xv) <= 2.0 ** -4 * np.abs(xv) + 2.0 ** -10 * scale)
    # exact: every decoded value is an e4m3 value times its block's power of two
    assert np.array_equal(dec, E4M3FN_VALUES[rows[:, :512]] * scale)


def test_single_token_gives_its_448_latent_dims():
    """(b) through a 528-byte cache: one token, o is its first 448 decoded
    values (the latent; dims 448..511 are RoPE), lse its score."""
    row, want = _golden_row()
    kv = np.zeros((1, 64, 528), dtype=np.uint8)
    kv[0, 0] = row
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 1, 3, 512))
    o, lse = mla_decode_ref(q, kv, "fp8_528", block_table=np.zeros((1, 1), dtype=np.int64),
                            cache_seqlens=np.array([1]), softmax_scale=SCALE)
    vals = np.repeat(np.array(want), 32)
    assert o.shape == (1, 1, 3, 448)
    assert np.array_equal(o[0, 0], np.broadcast_to(vals[:448], (3, 448)))
    assert np.allclose(lse[0, 0], float(np.float32(SCALE)) * (q[0, 0] @ vals), rtol=0, atol=1e-12)


def test_absorbed_equals_unabsorbed_with_448_latent_dims():
    """(a) with a 448-dim latent and 64 RoPE dims: explicit per-head keys and
    values through torch's float64 attention equal the absorbed form."""
    rng = np.random.default_rng(8)
    h, dh, dc, dr, n = 3, 128, 448, 64, 90
    K = rng.standard_normal((n, dc + dr))
    W_UK = rng.standard_normal((h, dh, dc)) / math.sqrt(dc)
    W_UV = rng.standard_normal((h, dh, dc)) / math.sqrt(dc)
    qC, qR = rng.standard_normal((h, dh)), rng.standard_normal((h, dr))
    q_abs = np.concatenate([np.einsum("hdc,hd->hc", W_UK, qC), qR], axis=1)
    o_lat, lse = attend(q_abs, K, SCALE, 448)
    for hh in range(h):
        k = np.concatenate([K[:, :dc] @ W_UK[hh].T, K[:, dc:]], axis=1)
        v = K[:, :dc] @ W_UV[hh].T
        qf = np.concatenate([qC[hh], qR[hh]])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qf)[None, None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
            scale=SCALE)[0, 0].numpy()
        assert np.max(np.abs(W_UV[hh] @ o_lat[hh] - ref)) < 1e-10
        assert abs(lse[hh] - torch.logsumexp(torch.from_numpy(k) @ torch.from_numpy(qf) * SCALE, 0).item()) < 1e-10


def test_528_workload_shapes_and_query_width_check():
    w = make_workload(batch=2, s_q=1, h_q=4, seqlens=[70, 3], kv_format="fp8_528", seed=1)
    assert tuple(w.q.shape) == (2, 1, 4, 512) and tuple(w.kv.shape) == (3, 64, 528)
    q = w.q.view(torch.int16).numpy().view(np.uint16)
    o, _ = mla_decode_ref(q, w.kv.numpy(), "fp8_528", block_table=w.block_table.numpy(),
                          cache_seqlens=w.cache_seqlens.numpy(), softmax_scale=SCALE)
    assert o.shape == (2, 1, 4, 448) and np.all(np.isfinite(o))
    with pytest.raises(ValueError):   # a 576-dim query against 512-dim keys
        mla_decode_ref(np.zeros((2, 1, 4, 576)), w.kv.numpy(), "fp8_528", block_table=w.block_table.numpy(),
                       cache_seqlens=w.cache_seqlens.numpy(), softmax_scale=SCALE)
