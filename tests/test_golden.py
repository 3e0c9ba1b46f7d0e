"""The oracle must keep reproducing its stored tiny-case outputs (guards its arithmetic
against unnoticed change); the same fixtures feed a GPU parity test."""
import importlib.util
import json
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def load_golden():
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "golden", "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(os.path.join(HERE, "golden", "tiny_cases.json")) as f:
        data = json.load(f)
    return mod, data["cases"]


def test_oracle_reproduces_golden():
    mod, cases = load_golden()
    assert len(cases) == 3
    for c in cases:
        q, k, v = mod.golden_inputs(c)
        kv = None if c["kv_len"] is None else np.array(c["kv_len"])
        O = oracle.attention_fp64(q, k, v, c["scale"], c["causal"], kv, kind="f32")
        np.testing.assert_allclose(O.reshape(-1), np.array(c["expected"]), rtol=0, atol=1e-14)
