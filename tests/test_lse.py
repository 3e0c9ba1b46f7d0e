"""GPU parity of the log-sum-exp side output (attn_fwd_lse, attn_fwd_f32_lse)
against the fp64 oracle, through the C ABI.

Tolerance (absolute, on the natural-log value): the bf16 path sums the bf16
rounded probabilities, each within 2^-9 relative of the exact value, so the sum
is within 2^-9 relative and the log within 2^-9 < 2e-3; the fp32 path is within
1e-5.  Rows without a visible key must be -inf exactly.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_long_sequence_amd import attnio
from exact_long_sequence_amd.inputs import WORKLOADS, make_inputs, oracle_view, sample_rows, workload_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
LSE_TOL = {"bf16": 2e-3, "f32": 1e-5}


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check_lse(got, want, dtype, label):
    got = np.asarray(got, dtype=np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(want)), f"{label}: -inf rows differ"
    fin = np.isfinite(want)
    assert np.isfinite(got[fin]).all(), f"{label}: non-finite lse on a row with visible keys"
    err = np.abs(got[fin] - want[fin])
    mx = float(err.max(initial=0.0))
    assert mx <= LSE_TOL[dtype], f"{label}: lse max_err={mx:.3e} (tol {LSE_TOL[dtype]})"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_lse_small_sweep(dtype, d, causal, padded):
    fwd = attnio.attn_fwd if dtype == "bf16" else attnio.attn_fwd_f32
    fwd_lse = attnio.attn_fwd_lse if dtype == "bf16" else attnio.attn_fwd_f32_lse
    kind = "bf16" if dtype == "bf16" else "f32"
    for N in (1, 65, 300, 1000):
        seed = 501 + N + 3 * d + 7 * causal + 11 * padded
        q, k, v, kv = make_inputs(2, 3, N, d, dtype, seed, padded=padded, kv_lo=0 if padded else None)
        scale = float(np.float32(1.0 / math.sqrt(d)))
        _log(f"lse sweep dtype={dtype} d={d} causal={causal} padded={padded} N={N} seed={seed}")
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        kvd = None if kv is None else kv.to(DEV)
        o, lse = fwd_lse(qd, kd, vd, causal=causal, kv_len=kvd, scale=scale)
        o_plain = fwd(qd, kd, vd, causal=causal, kv_len=kvd, scale=scale)
        torch.cuda.synchronize()
        bits = torch.int16 if dtype == "bf16" else torch.int32
        assert torch.equal(o.view(bits), o_plain.view(bits)), "O differs between attn_fwd and attn_fwd_lse"
        want = oracle.attention_lse_fp64(oracle_view(q), oracle_view(k), oracle_view(v), scale, causal,
                                         None if kv is None else kv.numpy(), kind=kind)
        _check_lse(lse.cpu().numpy(), want, dtype, f"N={N}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_lse_negative_scale(dtype, d):
    # the kernels' negative-scale instantiation (row minimum of the raw scores)
    fwd_lse = attnio.attn_fwd_lse if dtype == "bf16" else attnio.attn_fwd_f32_lse
    kind = "bf16" if dtype == "bf16" else "f32"
    for causal in (False, True):
        q, k, v, kv = make_inputs(2, 3, 300, d, dtype, 531 + d + causal, padded=True, kv_lo=0)
        scale = -float(np.float32(0.8 / math.sqrt(d)))
        _log(f"lse negative scale dtype={dtype} d={d} causal={causal}")
        o, lse = fwd_lse(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, kv_len=kv.to(DEV), scale=scale)
        torch.cuda.synchronize()
        want = oracle.attention_lse_fp64(oracle_view(q), oracle_view(k), oracle_view(v), scale, causal,
                                         kv.numpy(), kind=kind)
        _check_lse(lse.cpu().numpy(), want, dtype, f"negative scale causal={causal}")


def test_lse_headline_workload_sampled():
    w = WORKLOADS["bf16_causal_h32_n32k_d128"]
    _log("lse headline: inputs")
    q, k, v, kv = workload_inputs(w)
    o, lse = attnio.attn_fwd_lse(q.to(DEV), k.to(DEV), v.to(DEV), causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    rows = sample_rows(w.B, w.H, w.N, 512, seed=w.seed)
    _log(f"lse headline: oracle on {rows.size} rows")
    want = oracle.attention_lse_fp64(oracle_view(q), oracle_view(k), oracle_view(v), w.scale, w.causal,
                                     None, kind="bf16", rows=rows)
    got = lse.reshape(-1)[torch.as_tensor(rows, device=DEV)].cpu().numpy()
    _check_lse(got, want, "bf16", "headline")


def test_lse_empty_rows_and_binding_errors():
    q, k, v, _ = make_inputs(2, 1, 40, 64, "bf16", 77)
    kv = torch.tensor([0, 17], dtype=torch.int32)
    o, lse = attnio.attn_fwd_lse(q.to(DEV), k.to(DEV), v.to(DEV), kv_len=kv)
    torch.cuda.synchronize()
    assert torch.isneginf(lse[0]).all() and torch.isfinite(lse[1]).all()
    with pytest.raises(ValueError):
        attnio.attn_fwd_lse(q.to(DEV), k.to(DEV), v.to(DEV), lse=torch.empty(3, device=DEV))
