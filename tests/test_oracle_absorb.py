"""Pins for the oracle's absorption products (CPU only).

Composed with the oracle's decode, absorb_q and unabsorb_o must reproduce
multi-head attention written out with explicit per-head keys and values and
run through torch's attention (float64); hand-built weights pin the
orientation of each product.
"""

import math

import numpy as np
import torch

from oracle import mla_decode_ref
from oracle.absorb import absorb_q, unabsorb_o

SCALE = float(np.float32(576 ** -0.5))


def _bf16(x: np.ndarray) -> np.ndarray:
    """float64 values rounded to bf16, returned as bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _vals(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def test_absorbed_layer_equals_explicit_multi_head_attention():
    rng = np.random.default_rng(21)
    T, H, L = 3, 4, 130
    w_uk = _bf16(rng.standard_normal((H, 128, 512)) / math.sqrt(512))
    w_uv = _bf16(rng.standard_normal((H, 128, 512)) / math.sqrt(512))
    q_nope = _bf16(rng.standard_normal((T, H, 128)))
    q_rope = _bf16(rng.standard_normal((T, H, 64)))
    cache = _bf16(rng.standard_normal((L, 576)))            # [latent c ; rope k^R] per token
    q_abs = absorb_q(q_nope, q_rope, w_uk)                     # [T, H, 576]
    # attention over one unpaged sequence of L tokens (identity page table)
    pages = (L + 63) // 64
    rows = np.zeros((pages * 64, 576))
    rows[:L] = _vals(cache)
    o_lat, lse = mla_decode_ref(q_abs[:, None], rows, "bf16", block_table=np.tile(np.arange(pages), (T, 1)),
                                cache_seqlens=np.full(T, L), softmax_scale=SCALE, kv_is_decoded=True)
    out = unabsorb_o(o_lat[:, 0], w_uv)                         # [T, H, 128]
    c, kR = _vals(cache)[:, :512], _vals(cache)[:, 512:]
    for h in range(H):
        k = np.concatenate([c @ _vals(w_uk[h]).T, kR], axis=1)  # explicit keys [L, 192]
        v = c @ _vals(w_uv[h]).T                                # explicit values [L, 128]
        qf = np.concatenate([_vals(q_nope[:, h]), _vals(q_rope[:, h])], axis=1)  # [T, 192]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qf)[:, None], torch.from_numpy(k)[None].expand(T, L, 192),
            torch.from_numpy(v)[None].expand(T, L, 128), scale=SCALE)[:, 0].numpy()
        assert np.max(np.abs(out[:, h] - ref)) < 1e-10
        s = torch.from_numpy(qf) @ torch.from_numpy(k).T * SCALE
        assert np.max(np.abs(lse[:, 0, h] - torch.logsumexp(s, 1).numpy())) < 1e-10


def test_hand_built_weights_fix_the_orientation():
    # head 0: W^UK maps latent dim j to key dim j (j < 128), so q~ copies q^C into the first 128 latent
    # dims; head 1: key dim j reads latent dim 511 - j with weight 2, so q~[511 - j] = 2 q^C[j]
    T, H = 2, 2
    w_uk = np.zeros((H, 128, 512))
    w_uk[0, np.arange(128), np.arange(128)] = 1.0
    w_uk[1, np.arange(128), 511 - np.arange(128)] = 2.0
    rng = np.random.default_rng(3)
    q_nope = rng.standard_normal((T, H, 128))
    q_rope = rng.standard_normal((T, H, 64))
    q = absorb_q(q_nope, q_rope, w_uk)
    assert np.array_equal(q[:, 0, :128], q_nope[:, 0]) and not q[:, 0, 128:512].any()
    assert np.array_equal(q[:, 1, 511 - np.arange(128)], 2 * q_nope[:, 1]) and not q[:, 1, :384].any()
    assert np.array_equal(q[:, :, 512:], q_rope)
    # W^UV: head 0 output j = latent 4j; head 1 output j = -latent (j + 384)
    w_uv = np.zeros((H, 128, 512))
    w_uv[0, np.arange(128), 4 * np.arange(128)] = 1.0
    w_uv[1, np.arange(128), np.arange(128) + 384] = -1.0
    o = rng.standard_normal((T, H, 512))
    out = unabsorb_o(o, w_uv)
    assert np.array_equal(out[:, 0], o[:, 0, ::4])
    assert np.array_equal(out[:, 1], -o[:, 1, 384:])


def test_bf16_bit_patterns_and_values_agree():
    rng = np.random.default_rng(4)
    bits = _bf16(rng.standard_normal((2, 3, 128)))
    w = _bf16(rng.standard_normal((3, 128, 512)))
    rope = _bf16(rng.standard_normal((2, 3, 64)))
    assert np.array_equal(absorb_q(bits, rope, w), absorb_q(_vals(bits), _vals(rope), _vals(w)))
