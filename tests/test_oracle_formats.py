"""Pins for the oracle's number formats and cache-row decoding (CPU only)."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import E4M3FN_VALUES, bf16_bits_to_f64, decode_rows, f32_to_bf16_bits
from workload import quantize_fp8_656

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_e4m3fn_golden_codes():
    g = _load("e4m3fn_codes.json")["codes"]
    for hexcode, val in g.items():
        got = E4M3FN_VALUES[int(hexcode, 16)]
        if val == "nan":
            assert math.isnan(got), hexcode
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hexcode


def test_e4m3fn_all_codes_match_torch():
    # library cross-check: torch's float8_e4m3fn decode of every code
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ref) & np.isnan(E4M3FN_VALUES)
    assert np.all(both_nan | (ref == E4M3FN_VALUES))
    assert np.sum(np.isnan(E4M3FN_VALUES)) == 2
    assert np.nanmax(E4M3FN_VALUES) == 448.0


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    edges = np.array([0x3F808000, 0x3F818000, 0x3F80FFFF, 0x7F7FFFFF, 0x00008000, 0x80000000,
                      0x7F800000, 0xFF800000, 0x7FC00001, 0x3F7FFFFF], dtype=np.uint32)
    bits = np.concatenate([edges, bits])
    x = bits.view(np.float32)
    mine = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(mine[~nan], ref[~nan])
    # NaN stays NaN
    assert np.all(np.isnan(bf16_bits_to_f64(mine[nan])))


def test_bf16_bits_to_f64_exact():
    t = torch.randn(10000, dtype=torch.float32).to(torch.bfloat16)
    mine = bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(mine, t.to(torch.float64).numpy())


def test_fp8_row_golden():
    g = _load("fp8_row_656.json")
    row = np.zeros(656, dtype=np.uint8)
    for gi, c in enumerate(g["row"]["codes_per_group"]):
        row[gi * 128:(gi + 1) * 128] = int(c, 16)
    scales = np.array([int(h, 16) for h in g["row"]["scales_f32_hex"]], dtype=np.uint32)
    row[512:528] = scales.view(np.uint8)
    rope = np.full(64, 0x3F80, dtype=np.uint16)
    rope[:4] = [int(h, 16) for h in g["row"]["rope_bf16_hex_first4"]]
    row[528:656] = rope.view(np.uint8)
    vals = decode_rows(row[None, :], "fp8")[0]
    for gi, v in enumerate(g["expected_latent_per_group"]):
        assert np.all(vals[gi * 128:(gi + 1) * 128] == v), gi
    assert list(vals[512:516]) == g["expected_rope_first4"]
    assert np.all(vals[516:] == 1.0)


def test_bf16_row_decode_matches_view():
    t = torch.randn(7, 576).to(torch.bfloat16)
    rows = t.view(torch.uint8).numpy().reshape(7, 1152)
    assert np.array_equal(decode_rows(rows, "bf16"), t.to(torch.float64).numpy())


def test_fp8_decode_within_quantisation_bound():
    """Writer (torch cast) then oracle decode stays within e4m3's error bound.

    e4m3 keeps 3 mantissa bits, so rounding a normal value errs by at most 2^-4
    of it (walkthrough §三: relative error about 2^-4); subnormals err by at
    most half their spacing, 2^-10 in scaled units; the final bf16 rounding adds
    at most 2^-9 relative. A decode that applied the wrong group's scale, read
    the scales or rope from the wrong bytes, or dropped the scale, fails this.
    """
    g = torch.Generator().manual_seed(3)
    n = 512
    latent = torch.randn(n, 512, generator=g) * torch.exp(torch.randn(n, 4, generator=g)).repeat_interleave(128, 1)
    latent[0, :128] = 0.0  # an all-zero group (scale 1)
    latent[1, 128:256] *= 1e-3
    rope = torch.randn(n, 64, generator=g).to(torch.bfloat16)
    rows = quantize_fp8_656(latent, rope).numpy()
    dec = decode_rows(rows, "fp8")
    x = latent.to(torch.float64).numpy()
    scale = np.repeat(rows[:, 512:528].copy().view("<f4").reshape(n, 4).astype(np.float64), 128, axis=1)
    bound = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * scale + 2.0 ** -8 * np.abs(x) + 1e-30
    assert np.all(np.abs(dec[:, :512] - x) <= bound)
    assert np.array_equal(dec[:, 512:], rope.to(torch.float64).numpy())
    # the bound is tight enough to catch a swapped scale group
    wrong = dec[:, :512].reshape(n, 4, 128)[:, ::-1].reshape(n, 512)
    assert np.mean(np.abs(wrong - x) <= bound) < 0.9
