"""Pins for the oracle's FP8 cache writer (quantise on write).

The oracle decides e4m3 rounding by nearest value in its own table; these
tests hold it to torch's e4m3fn cast (an independent implementation), to hand
worked rows and tie cases, to the input generator's torch writer, and to
e4m3's error bound.
"""

import json
import os

import numpy as np
import torch

from oracle import append_rows, decode_rows, f32_to_e4m3fn_codes, quantize_rows
from workload.gen import quantize_fp8_656

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_quantize_row.json")


def _bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).contiguous().view(torch.int16).numpy().view(np.uint16)


def test_codes_match_torch_cast_on_every_bf16_value_in_range():
    # every bf16 bit pattern whose value is finite with |x| <= 448 (this holds every e4m3 tie point)
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448)
    vals = vals[keep]
    want = torch.from_numpy(vals.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f32_to_e4m3fn_codes(vals), want)


def test_codes_match_torch_cast_on_random_fp32():
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-14, np.log2(448), 400_000)).astype(np.float32)
    vals = np.where(rng.random(mag.size) < 0.5, -mag, mag).astype(np.float32)
    vals = np.clip(vals, -448, 448)
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f32_to_e4m3fn_codes(vals), want)


def test_hand_worked_ties_and_signs():
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 15 * 2.0 ** -10: 0x08,
             432.0: 0x7E, 440.0: 0x7E, 416.0: 0x7D, -0.0: 0x80, -(2.0 ** -11): 0x80, 448.0: 0x7E, -448.0: 0xFE}
    got = f32_to_e4m3fn_codes(np.array(list(cases), dtype=np.float32))
    assert [int(c) for c in got] == list(cases.values())


def _golden_row():
    g = json.load(open(GOLDEN))
    latent = np.zeros(512, dtype=np.float32)
    for k, v in g["input_latent_nonzero"].items():
        latent[int(k)] = v
    rope_bits = np.full(64, 0x3F80, dtype=np.uint16)
    rope_bits[:4] = [int(h, 16) for h in g["input_rope_bf16_hex_first4"]]
    src = np.concatenate([_bf16_bits(torch.from_numpy(latent)), rope_bits])
    return g, src


def test_golden_row():
    g, src = _golden_row()
    row = quantize_rows(src[None, :])[0]
    codes = np.zeros(512, dtype=np.uint8)
    for k, v in g["expected_codes_nonzero"].items():
        codes[int(k)] = int(v, 16)
    assert np.array_equal(row[:512], codes)
    scales = row[512:528].copy().view("<u4")
    assert [int(s) for s in scales] == [int(h, 16) for h in g["expected_scales_f32_hex"]]
    assert np.array_equal(row[528:].copy().view("<u2"), src[512:])


def test_matches_the_input_generators_writer():
    gen = torch.Generator().manual_seed(11)
    n = 300
    latent = torch.randn(n, 512, generator=gen) * torch.exp(2 * torch.randn(n, 4, generator=gen)).repeat_interleave(128, 1)
    latent = latent.to(torch.bfloat16)
    latent[0, :128] = 0
    latent[1, 256:384] = -latent[1, 256:384].abs()
    rope = torch.randn(n, 64, generator=gen).to(torch.bfloat16)
    src = np.concatenate([_bf16_bits(latent), _bf16_bits(rope)], axis=1)
    assert np.array_equal(quantize_rows(src), quantize_fp8_656(latent.float(), rope).numpy())


def test_round_trip_within_e4m3_bound():
    gen = torch.Generator().manual_seed(5)
    n = 256
    latent = (torch.randn(n, 512, generator=gen) * torch.exp(torch.randn(n, 4, generator=gen)).repeat_interleave(128, 1))
    src = np.concatenate([_bf16_bits(latent), _bf16_bits(torch.randn(n, 64, generator=gen))], axis=1)
    rows = quantize_rows(src)
    x = (src[:, :512].astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    dec = decode_rows(rows, "fp8")
    scale = np.repeat(rows[:, 512:528].copy().view("<f4").astype(np.float64), 128, axis=1)
    # 3 mantissa bits: a normal value errs by at most 2^-4 of itself; subnormals by half their spacing,
    # 2^-10 in scaled units; the bf16 rounding of the decoded value adds at most 2^-8 relative
    bound = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * scale + 2.0 ** -8 * np.abs(x) + 1e-30
    assert np.all(np.abs(dec[:, :512] - x) <= bound)
    # the largest magnitude of each group lands on 448 * scale (up to the fp32 rounding of the scale)
    amax = np.abs(x).reshape(n, 4, 128).max(axis=2)
    top = np.abs(dec[:, :512]).reshape(n, 4, 128).max(axis=2)
    assert np.allclose(top, amax, rtol=2.0 ** -7)


def test_append_writes_only_valid_distinct_slots():
    rng = np.random.default_rng(2)
    num_rows = 5 * 64
    cache = rng.integers(0, 256, (num_rows, 656), dtype=np.uint8)
    n = 40
    src = _bf16_bits(torch.from_numpy(rng.standard_normal((n, 576)).astype(np.float32)))
    slots = rng.permutation(num_rows)[:n].astype(np.int64)
    slots[3] = -1
    slots[7] = num_rows          # one past the end
    slots[9] = -5
    out = append_rows(cache, slots, src)
    rows = quantize_rows(src)
    written = np.zeros(num_rows, dtype=bool)
    for i, s in enumerate(slots):
        if 0 <= s < num_rows:
            assert np.array_equal(out[s], rows[i])
            written[s] = True
    assert np.array_equal(out[~written], cache[~written])
    assert written.sum() == n - 3
