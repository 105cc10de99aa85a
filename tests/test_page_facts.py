"""Layout and cost facts printed on the pages, checked against the constants
the oracle and the input writer use (CPU only)."""

import json
import os

import numpy as np

import oracle.mla_oracle as om
from workload import D_QK, D_ROPE, D_V, ROW_BYTES

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_page_facts():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        facts = {x["name"]: x for x in json.load(f)["facts"]}
    computed = {
        "bf16 row bytes": D_QK * 2,
        "fp8 row bytes": D_V * 1 + 4 * 4 + D_ROPE * 2,
        "fp8 saving fraction": 1 - 656 / 1152,
        "128K x 62 layers bf16 GiB": 131072 * 62 * 1152 / 2 ** 30,
        "128K x 62 layers fp8 GiB": 131072 * 62 * 656 / 2 ** 30,
        "MHA bytes per token per layer": 128 * 128 * 2 * 2,
        "MLA bf16 ratio to MHA": 65536 / 1152,
        "64x512 fp32 output registers": 64 * 512 * 4 // 4,
        "decode FLOPs per (query row, token)": 2 * (om.D_QK + om.D_V),
        "decode bytes per token bf16": 2 * om.D_QK,
        "fp8 528 row bytes": om.FORMATS["fp8_528"][1] * 1 + (om.FORMATS["fp8_528"][1] // om.MX_BLOCK) * 1,
        "MLA 528 ratio to MHA": 65536 / 528,
    }
    for name, val in computed.items():
        f = facts[name]
        assert abs(val - f["value"]) <= f.get("tol", 0), (name, val, f)
    assert ROW_BYTES == {"bf16": facts["bf16 row bytes"]["value"], "fp8": facts["fp8 row bytes"]["value"],
                         "fp8_528": facts["fp8 528 row bytes"]["value"]}
    assert {k: v[0] for k, v in om.FORMATS.items()} == ROW_BYTES
    assert om.D_QK == D_QK == 576 and om.D_V == D_V == 512 and om.BLOCK_SIZE == 64
