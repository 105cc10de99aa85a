"""Seeded random shapes through the whole decode path against the float64 oracle.

Each case draws batch, query positions, head count (including counts that pad
a row group, and with several query positions row groups that span positions),
cache format, dense/causal/sparse, sequence lengths (including
empty and one-token sequences) and the number of parts (including fewer parts
than row-group sequences, which selects the combine's wide mapping), then
compares every query row with the oracle at the stated tolerances.
"""

import numpy as np
import pytest

from workload import make_workload

from tests.gpu_helpers import compare, oracle, run_gpu, say, workload_floor_fn

pytestmark = pytest.mark.gpu


def _cases(n=32, seed=2024, s_qs=(1, 1, 2, 3), h_qs=(1, 8, 16, 17, 33, 64, 65, 100, 128, 129, 200),
           fmts=("bf16", "fp8"), modes=("dense", "dense", "causal", "sparse"), tag="fuzz", max_len=700):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        batch = int(rng.integers(1, 7))
        s_q = int(rng.choice(list(s_qs)))
        h_q = int(rng.choice(list(h_qs)))
        fmt = str(rng.choice(list(fmts)))
        mode = str(rng.choice(list(modes)))
        num_parts = rng.choice([0, 1, 5, 64, 300])
        kw = dict(batch=batch, s_q=s_q, h_q=h_q, kv_format=fmt, seed=int(rng.integers(0, 1 << 30)))
        if mode == "sparse":
            tokens = int(rng.choice([64, 128, 512]))
            topk = int(rng.choice([1, 63, 64, 65, 100]))
            topk = min(topk, tokens - s_q + 1)
            kw.update(topk=topk, sparse_tokens_per_seq=tokens, invalid_frac=float(rng.choice([0.0, 0.05, 0.5])))
        else:
            lens = rng.integers(0, max_len, batch)
            lens[rng.random(batch) < 0.15] = 0
            lens[rng.random(batch) < 0.15] = 1
            kw.update(seqlens=[int(x) for x in lens], causal=(mode == "causal"))
        out.append((f"{tag}{k}-{fmt}-{mode}-B{batch}-s{s_q}-h{h_q}-P{int(num_parts)}", kw,
                    None if num_parts == 0 else int(num_parts)))
    return out


# the first draw as it always was, then causal-heavy shapes with several query
# positions (row groups that span positions, every format, 528-byte rows too),
# then causal calls whose sequences are shorter than their query positions
# (the first positions of a row group see no token)
CASES = _cases() + _cases(n=24, seed=2026, s_qs=(2, 3, 4), h_qs=(3, 4, 5, 12, 20, 24, 40, 48, 96),
                          fmts=("bf16", "fp8", "fp8_528"), modes=("causal", "causal", "dense", "sparse"),
                          tag="fuzzpos") + \
    _cases(n=24, seed=2027, s_qs=(3, 5, 8, 13), h_qs=(1, 2, 3, 6, 7, 10, 20, 30), fmts=("bf16", "fp8", "fp8_528"),
           modes=("causal",), tag="fuzzshort", max_len=24)


@pytest.mark.parametrize("label,kw,num_parts", CASES, ids=[c[0] for c in CASES])
def test_random_shapes_match_oracle(label, kw, num_parts):
    say(f"case: {label} {kw.get('seqlens', kw.get('topk'))}")
    w = make_workload(name=label, **kw)
    o, lse, _, _ = run_gpu(w, num_parts=num_parts)
    o_ref, lse_ref = oracle(w)
    compare(o, lse, o_ref, lse_ref, None, label, floor_fn=workload_floor_fn(w))
