"""Reference for the absorption products on either side of the decode.

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the GPU path.

Page cited: [Walkthrough] "矩阵、注意力与 GPU：拆解 DeepGEMM 与 FlashMLA"
(msy.plus), §六, the absorption passage and "结果：decode 变成 MQA": per head
i, the key up-projection W^UK_i (d_h x d_c = 128 x 512) folds into the query,
q~_i = W^UK_i^T q^C_i, so the score against a cached latent c is q~_i . c
plus the RoPE term; the value up-projection W^UV_i (128 x 512) is applied
after the weighted sum of latents, o_i = W^UV_i (sum_j p_ij c_j).

What is computed (float64, from bf16 inputs):
  * absorb_q: q[t, i] = [W^UK_i^T q^C[t, i] ; q^R[t, i]], 576 values, the
    decode's query row (latent part first, RoPE part copied);
  * unabsorb_o: out[t, i] = W^UV_i o_lat[t, i], 128 values per head.

Reading where the page is silent: the RoPE part
of the query is passed in already rotated; the absorbed query's first 512
values are the latent dims and the last 64 the RoPE dims, the order of the
cache row.
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import bf16_bits_to_f64

D_NOPE = 128
D_C = 512
D_ROPE = 64


def _values(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    return bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def absorb_q(q_nope: np.ndarray, q_rope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """q_nope [T, H, 128], q_rope [T, H, 64], W^UK [H, 128, 512] -> absorbed queries [T, H, 576].

    Arrays of uint16 are bf16 bit patterns; anything else is taken as values.
    """
    qn, qr, w = _values(q_nope), _values(q_rope), _values(w_uk)
    T, H, dn = qn.shape
    if dn != D_NOPE or qr.shape != (T, H, D_ROPE) or w.shape != (H, D_NOPE, D_C):
        raise ValueError("absorb_q takes q_nope [T, H, 128], q_rope [T, H, 64], w_uk [H, 128, 512]")
    out = np.empty((T, H, D_C + D_ROPE))
    for i in range(H):
        out[:, i, :D_C] = qn[:, i, :] @ w[i]     # row form of W^UK_i^T q^C_i
    out[:, :, D_C:] = qr
    return out


def unabsorb_o(o_lat: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """Latent attention outputs [T, H, 512], W^UV [H, 128, 512] -> per-head outputs [T, H, 128]."""
    o, w = _values(o_lat), _values(w_uv)
    T, H, dc = o.shape
    if dc != D_C or w.shape != (H, D_NOPE, D_C):
        raise ValueError("unabsorb_o takes o_lat [T, H, 512], w_uv [H, 128, 512]")
    out = np.empty((T, H, D_NOPE))
    for i in range(H):
        out[:, i, :] = o[:, i, :] @ w[i].T       # row form of W^UV_i o_i
    return out
