"""GPU parity: the HIP path against the fp64 oracle, through the C ABI.

Small shapes are checked on every output row and span several query / key
tiles plus ragged tails; the full-size workloads are checked on every row
(when the oracle finishes in seconds) or on a seeded sample of at least 4096
rows plus boundary rows, in the launch configuration the benchmark times.
"""

import json
import math
import os
import sys

import numpy as np
import pytest
import torch

from exact_long_sequence_amd.inputs import WORKLOADS, make_inputs, sample_rows, workload_inputs

from .parity_util import compare, gpu_rows, oracle_rows, run_gpu

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SMALL_N = [1, 2, 63, 64, 65, 127, 129, 1000, 1024]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_small_sweep_every_row(dtype, d, causal, padded):
    for N in SMALL_N:
        seed = 17 + N + 3 * d + 7 * causal + 11 * padded
        B, H = 2, 3
        q, k, v, kv_len = make_inputs(B, H, N, d, dtype, seed, padded=padded,
                                      kv_lo=0 if padded else None)
        scale = float(np.float32(1.0 / math.sqrt(d)))
        _log(f"small sweep dtype={dtype} d={d} causal={causal} padded={padded} N={N} seed={seed} "
             f"kv_len={None if kv_len is None else kv_len.tolist()}")
        out = run_gpu(q, k, v, causal, kv_len, scale, dtype)
        want = oracle_rows(q, k, v, causal, kv_len, scale, dtype)
        compare(gpu_rows(out), want, dtype, f"N={N}")


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity(name):
    w = WORKLOADS[name]
    _log(f"workload {name}: generating inputs")
    q, k, v, kv_len = workload_inputs(w)
    _log(f"workload {name}: running the HIP path")
    out = run_gpu(q, k, v, w.causal, kv_len, w.scale, w.dtype)
    if w.full_check:
        rows = None
    else:
        rows = sample_rows(w.B, w.H, w.N, 4096, w.seed, kv_len=None if kv_len is None else kv_len.numpy())
        assert rows.size >= 4096
    _log(f"workload {name}: oracle on {'all' if rows is None else rows.size} rows")
    want = oracle_rows(q, k, v, w.causal, kv_len, w.scale, w.dtype, rows)
    got = gpu_rows(out, rows)
    if rows is None:
        got, want = got.reshape(-1, w.d), want.reshape(-1, w.d)
    mx, mean = compare(got, want, w.dtype, name)
    _log(f"workload {name}: max_err={mx:.3e} mean_err={mean:.3e}")


def test_golden_tiny_cases():
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "golden", "tiny_cases.json")) as f:
        cases = json.load(f)["cases"]
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(here, "golden", "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    for c in cases:
        q, k, v = (torch.from_numpy(x) for x in mod.golden_inputs(c))
        kv = None if c["kv_len"] is None else torch.tensor(c["kv_len"], dtype=torch.int32)
        want = np.array(c["expected"]).reshape(q.shape)
        _log(f"golden {c['name']}")
        out = run_gpu(q, k, v, c["causal"], kv, c["scale"], "f32")
        compare(gpu_rows(out), want, "f32", c["name"])
        # the inputs are on a 1/8 grid, so they are exact in bf16 as well
        out = run_gpu(q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16),
                      c["causal"], kv, c["scale"], "bf16")
        compare(gpu_rows(out), want, "bf16", c["name"] + "/bf16")
