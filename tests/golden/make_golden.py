"""Writes tests/golden/tiny_cases.json.  Calls only the oracle.

Each case's inputs are regenerated from its seed by golden_inputs() below
(numpy PCG64, values on a 1/8 grid in [-2, 2], so every value is exact in bf16
and fp32); the stored numbers are the oracle's fp64 outputs.  The arithmetic
they follow is the attention operator graph (scores, optional mask, softmax,
weighted sum of values) of "From Attention Graph to FlashAttention - A
Memory-Centric Compilation Approach in AICF", section 1.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

CASES = [
    {"name": "causal_b1_h2_n7_d64", "B": 1, "H": 2, "N": 7, "d": 64, "causal": True,
     "kv_len": None, "scale": 0.125, "seed": 7},
    {"name": "padded_b2_h1_n5_d128", "B": 2, "H": 1, "N": 5, "d": 128, "causal": False,
     "kv_len": [2, 5], "scale": 0.08838834764831845, "seed": 8},
    {"name": "causal_padded_b2_h1_n6_d64_kv0", "B": 2, "H": 1, "N": 6, "d": 64, "causal": True,
     "kv_len": [0, 3], "scale": 0.5, "seed": 9},
]


def golden_inputs(case):
    rng = np.random.default_rng(case["seed"])
    shape = (case["B"], case["H"], case["N"], case["d"])
    return [rng.integers(-16, 17, size=shape).astype(np.float32) / np.float32(8) for _ in range(3)]


def main():
    out = {"about": "oracle fp64 outputs for tiny seeded cases; inputs from golden_inputs()",
           "cases": []}
    for c in CASES:
        q, k, v = golden_inputs(c)
        kv = None if c["kv_len"] is None else np.array(c["kv_len"])
        O = oracle.attention_fp64(q, k, v, c["scale"], c["causal"], kv, kind="f32")
        out["cases"].append(dict(c, expected=[float(x) for x in O.reshape(-1)]))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_cases.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
