"""Plant plausible mistakes in the oracle (CPU, monkeypatched) and check that
the pins catch each one. This guards the pins themselves: a pin that passes
on a broken oracle would prove nothing."""

import numpy as np
import pytest

import oracle.mla_oracle as om
import tests.test_oracle_attention as ta
import tests.test_oracle_formats as tf


def _attend_no_rope(q, K, scale, d_v=512):
    if K.shape[0] == 0:
        return np.zeros((q.shape[0], 512)), np.full(q.shape[0], -np.inf)
    S = (q[:, :512] @ K[:, :512].T) * scale
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return (E / l) @ K[:, :512], (m + np.log(l))[:, 0]


def _attend_wrong_value_slice(q, K, scale, d_v=512):
    if K.shape[0] == 0:
        return np.zeros((q.shape[0], 512)), np.full(q.shape[0], -np.inf)
    S = (q @ K.T) * scale
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return (E / l) @ K[:, 64:], (m + np.log(l))[:, 0]


def _attend_lse_without_max(q, K, scale, d_v=512):
    if K.shape[0] == 0:
        return np.zeros((q.shape[0], 512)), np.full(q.shape[0], -np.inf)
    S = (q @ K.T) * scale
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return (E / l) @ K[:, :512], np.log(l)[:, 0]


_real_attended_rows = om.attended_rows


def _rows_causal_off_by_one(b, i, *, s_q, num_rows, block_table, cache_seqlens, causal, indices):
    if causal and indices is None:
        L = int(cache_seqlens[b])
        t = np.arange(max(0, L - s_q + i))
        return np.asarray(block_table[b])[t // 64] * 64 + t % 64
    return _real_attended_rows(b, i, s_q=s_q, num_rows=num_rows, block_table=block_table,
                               cache_seqlens=cache_seqlens, causal=causal, indices=indices)


def _rows_ignore_block_table(b, i, *, s_q, num_rows, block_table, cache_seqlens, causal, indices):
    if indices is None:
        return np.arange(int(cache_seqlens[b]))
    return _real_attended_rows(b, i, s_q=s_q, num_rows=num_rows, block_table=block_table,
                               cache_seqlens=cache_seqlens, causal=causal, indices=indices)


def _rows_keep_minus_one(b, i, *, s_q, num_rows, block_table, cache_seqlens, causal, indices):
    if indices is not None:
        idx = np.asarray(indices[b, i], dtype=np.int64)
        return idx[idx < num_rows]  # forgets to drop -1 (reads the last row)
    return _real_attended_rows(b, i, s_q=s_q, num_rows=num_rows, block_table=block_table,
                               cache_seqlens=cache_seqlens, causal=causal, indices=indices)


def _rows_wrap_invalid_pages(b, i, *, s_q, num_rows, block_table, cache_seqlens, causal, indices):
    if indices is None:
        L = int(cache_seqlens[b])
        t = np.arange(L)
        pages = np.asarray(block_table[b])[np.minimum(t // 64, len(block_table[b]) - 1)]
        return (pages % (num_rows // 64)) * 64 + t % 64  # reads some page for -1 / out-of-pool ids
    return _real_attended_rows(b, i, s_q=s_q, num_rows=num_rows, block_table=block_table,
                               cache_seqlens=cache_seqlens, causal=causal, indices=indices)


def _rows_past_table_reuse_last_page(b, i, *, s_q, num_rows, block_table, cache_seqlens, causal, indices):
    if indices is None and not causal:
        L = int(cache_seqlens[b])
        t = np.arange(L)
        table = np.asarray(block_table[b])
        pages = table[np.minimum(t // 64, len(table) - 1)]
        keep = (pages >= 0) & (pages < num_rows // 64)
        return pages[keep] * 64 + t[keep] % 64
    return _real_attended_rows(b, i, s_q=s_q, num_rows=num_rows, block_table=block_table,
                               cache_seqlens=cache_seqlens, causal=causal, indices=indices)


_real_decode = om.decode_rows


def _decode_scale_per_64(rows, kv_format):
    out = _real_decode(rows, kv_format)
    if kv_format != "fp8":
        return out
    n = rows.shape[0]
    codes = om.E4M3FN_VALUES[rows[:, :512]].astype(np.float32)
    scales = rows[:, 512:528].copy().view("<f4").reshape(n, 4)
    sc = np.repeat(np.tile(scales, 2), 64, axis=1).astype(np.float32)  # wrong group width
    out[:, :512] = om.bf16_bits_to_f64(om.f32_to_bf16_bits(codes * sc))
    return out


def _bf16_truncate(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


ATTENTION_PINS = [
    ta.test_absorbed_equals_unabsorbed_mha,
    ta.test_single_token_returns_its_latent,
    ta.test_equal_scores_give_mean_of_latents,
    ta.test_split_merge_identity,
    ta.test_causal_alignment,
    ta.test_page_permutation_invariance,
    ta.test_sparse_all_rows_equals_dense_and_ignores_invalid,
    ta.test_invalid_pages_and_positions_past_the_table_are_skipped,
]


@pytest.mark.parametrize("mutant", [_attend_no_rope, _attend_wrong_value_slice, _attend_lse_without_max])
def test_attend_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(om, "attend", mutant)
    monkeypatch.setattr(ta, "attend", mutant)
    assert any(_fails(p) for p in ATTENTION_PINS)


@pytest.mark.parametrize("mutant", [_rows_causal_off_by_one, _rows_ignore_block_table, _rows_keep_minus_one,
                                    _rows_wrap_invalid_pages, _rows_past_table_reuse_last_page])
def test_masking_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(om, "attended_rows", mutant)
    assert any(_fails(p) for p in ATTENTION_PINS)


def test_fp8_group_mutant_is_caught(monkeypatch):
    monkeypatch.setattr(om, "decode_rows", _decode_scale_per_64)
    monkeypatch.setattr(tf, "decode_rows", _decode_scale_per_64)
    assert _fails(tf.test_fp8_decode_within_quantisation_bound) or _fails(tf.test_fp8_row_golden)


def test_bf16_rounding_mutant_is_caught(monkeypatch):
    monkeypatch.setattr(tf, "f32_to_bf16_bits", _bf16_truncate)
    assert _fails(tf.test_bf16_rne_matches_torch)


# ---- the FP8 cache writer -------------------------------------------------

import oracle.quantize as oq  # noqa: E402
import tests.test_oracle_quantize as tq  # noqa: E402

_real_codes = oq.f32_to_e4m3fn_codes
_real_quantize = oq.quantize_rows


def _codes_ties_away(y):
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    hi = np.minimum(np.searchsorted(oq._POS_VALUES, a, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    pick_hi = (oq._POS_VALUES[hi] - a) <= (a - oq._POS_VALUES[lo])
    return np.where(pick_hi, hi, lo).astype(np.uint8) | (np.signbit(y).astype(np.uint8) << np.uint8(7))


def _codes_unsigned_zero(y):
    c = _real_codes(y)
    return np.where((c & 0x7F) == 0, np.uint8(0), c).astype(np.uint8)


def _quantize_scale_over_256(src):
    bits = np.asarray(src, dtype=np.uint16)
    n = bits.shape[0]
    lat = (bits[:, :512].astype(np.uint32) << np.uint32(16)).view(np.float32).reshape(n, 4, 128)
    amax = np.abs(lat).max(axis=2)
    scale = np.where(amax == 0, np.float32(1), amax / np.float32(256)).astype(np.float32)
    y = np.clip((lat / scale[:, :, None]).astype(np.float32), -448, 448)
    out = _real_quantize(bits)
    out[:, :512] = _real_codes(y).reshape(n, 512)
    out[:, 512:528] = scale.astype("<f4").view(np.uint8).reshape(n, 16)
    return out


def _quantize_scales_big_endian(src):
    out = _real_quantize(src)
    out[:, 512:528] = out[:, 512:528].reshape(-1, 4, 4)[:, :, ::-1].reshape(-1, 16)
    return out


def _quantize_rope_from_latent(src):
    out = _real_quantize(src)
    bits = np.asarray(src, dtype=np.uint16)
    out[:, 528:] = bits[:, :64].astype("<u2").view(np.uint8).reshape(-1, 128)
    return out


QUANTIZE_PINS = [tq.test_codes_match_torch_cast_on_every_bf16_value_in_range, tq.test_hand_worked_ties_and_signs,
                 tq.test_golden_row, tq.test_matches_the_input_generators_writer, tq.test_round_trip_within_e4m3_bound]


@pytest.mark.parametrize("mutant", [_codes_ties_away, _codes_unsigned_zero])
def test_e4m3_rounding_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(tq, "f32_to_e4m3fn_codes", mutant)
    monkeypatch.setattr(oq, "f32_to_e4m3fn_codes", mutant)
    assert any(_fails(p) for p in QUANTIZE_PINS)


@pytest.mark.parametrize("mutant", [_quantize_scale_over_256, _quantize_scales_big_endian, _quantize_rope_from_latent])
def test_writer_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(tq, "quantize_rows", mutant)
    assert any(_fails(p) for p in QUANTIZE_PINS)


# ---- the absorption products ---------------------------------------------

import oracle.absorb as oa  # noqa: E402
import tests.test_oracle_absorb as tab  # noqa: E402

_real_absorb = oa.absorb_q
_real_unabsorb = oa.unabsorb_o


def _absorb_next_heads_weights(q_nope, q_rope, w_uk):
    return _real_absorb(q_nope, q_rope, np.roll(np.asarray(w_uk), 1, axis=0))


def _absorb_rope_dropped(q_nope, q_rope, w_uk):
    out = _real_absorb(q_nope, q_rope, w_uk)
    out[:, :, 512:] = 0
    return out


def _unabsorb_reshaped_weights(o_lat, w_uv):
    w = oa._values(w_uv)
    return _real_unabsorb(o_lat, w.reshape(w.shape[0], 512, 128).transpose(0, 2, 1))


ABSORB_PINS = [tab.test_absorbed_layer_equals_explicit_multi_head_attention, tab.test_hand_built_weights_fix_the_orientation]


@pytest.mark.parametrize("mutant", [_absorb_next_heads_weights, _absorb_rope_dropped])
def test_absorb_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(tab, "absorb_q", mutant)
    assert any(_fails(p) for p in ABSORB_PINS)


def test_unabsorb_mutant_is_caught(monkeypatch):
    monkeypatch.setattr(tab, "unabsorb_o", _unabsorb_reshaped_weights)
    assert any(_fails(p) for p in ABSORB_PINS)


# ---- the 528-byte row -----------------------------------------------------

import tests.test_oracle_528 as t528  # noqa: E402


def _decode528_blocks_of_64(rows, kv_format):
    if kv_format != "fp8_528":
        return _real_decode(rows, kv_format)
    rows = np.ascontiguousarray(rows)
    vals = om.E4M3FN_VALUES[rows[:, :512]] * np.repeat(om.ue8m0_values(rows[:, 512:520]).astype(np.float64), 64, axis=1)
    return vals


def _decode528_bias_128(rows, kv_format):
    if kv_format != "fp8_528":
        return _real_decode(rows, kv_format)
    rows = np.ascontiguousarray(rows)
    return om.E4M3FN_VALUES[rows[:, :512]] * np.repeat(np.ldexp(1.0, rows[:, 512:].astype(np.int64) - 128), 32, axis=1)


def _decode528_scales_reversed(rows, kv_format):
    if kv_format != "fp8_528":
        return _real_decode(rows, kv_format)
    rows = np.array(rows, copy=True)
    rows[:, 512:] = rows[:, 512:][:, ::-1]
    return _real_decode(rows, kv_format)


_real_attend = om.attend


def _attend_value_from_the_end(q, K, scale, d_v=512):
    o, lse = _real_attend(q, K, scale, K.shape[1])
    return o[:, -d_v:], lse   # takes the last d_v dims (RoPE included) as the value


import oracle.quantize as oq528  # noqa: E402

_real_q528 = oq528.quantize_rows_528


def _q528_scale_rounded_down(src):
    out = _real_q528(src)
    bits = np.asarray(src, dtype=np.uint16)
    x = (bits.astype(np.uint32) << 16).view(np.float32).reshape(-1, 16, 32).astype(np.float64)
    amax = np.abs(x).max(axis=2)
    k = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0) / 448.0)), 0).astype(np.int64)
    y = np.clip(np.ldexp(x, -k[:, :, None]), -448, 448).astype(np.float32)
    out[:, :512] = oq528.f32_to_e4m3fn_codes(y).reshape(-1, 512)
    out[:, 512:] = (k + 127).astype(np.uint8)
    return out


def _q528_blocks_of_16(src):
    bits = np.asarray(src, dtype=np.uint16)
    n = bits.shape[0]
    x = (bits.astype(np.uint32) << 16).view(np.float32).reshape(n, 32, 16)
    amax = np.abs(x).max(axis=2)
    k = np.where(amax == 0, 0, oq528.ue8m0_exponent_for(np.where(amax == 0, 1.0, amax)))
    y = np.ldexp(x.astype(np.float64), -k[:, :, None]).astype(np.float32)
    out = np.empty((n, 528), dtype=np.uint8)
    out[:, :512] = oq528.f32_to_e4m3fn_codes(y).reshape(n, 512)
    out[:, 512:] = (k[:, ::2] + 127).astype(np.uint8)
    return out


PINS_528 = [t528.test_528_row_golden, t528.test_528_writer_golden, t528.test_528_round_trip_bound_and_generator_agreement,
            t528.test_528_scale_is_the_smallest_power_of_two_covering_amax, t528.test_single_token_gives_its_448_latent_dims,
            t528.test_absorbed_equals_unabsorbed_with_448_latent_dims]


@pytest.mark.parametrize("mutant", [_decode528_blocks_of_64, _decode528_bias_128, _decode528_scales_reversed])
def test_528_decode_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(om, "decode_rows", mutant)
    monkeypatch.setattr(t528, "decode_rows", mutant)
    assert any(_fails(p) for p in PINS_528)


def test_528_value_slice_mutant_is_caught(monkeypatch):
    monkeypatch.setattr(om, "attend", _attend_value_from_the_end)
    monkeypatch.setattr(t528, "attend", _attend_value_from_the_end)
    assert any(_fails(p) for p in PINS_528)


@pytest.mark.parametrize("mutant", [_q528_scale_rounded_down, _q528_blocks_of_16])
def test_528_writer_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(t528, "quantize_rows_528", mutant)
    assert any(_fails(p) for p in PINS_528)
