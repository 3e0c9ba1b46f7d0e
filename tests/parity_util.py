"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on the
same inputs, compare element by element with the stated tolerances."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from exact_long_sequence_amd import attnio
from exact_long_sequence_amd.inputs import oracle_view

# bf16 inputs, fp32 accumulation, bf16 output: max |err| <= 2e-2 and mean |err| <= 2e-3;
# fp32 end to end: max |err| <= 1e-4 (both against the fp64 oracle).
TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, None)}


def run_gpu(q, k, v, causal, kv_len, scale, dtype):
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    kvd = None if kv_len is None else kv_len.to(device=dev, dtype=torch.int32)
    fn = attnio.attn_fwd if dtype == "bf16" else attnio.attn_fwd_f32
    out = fn(qd, kd, vd, causal=causal, kv_len=kvd, scale=scale)
    torch.cuda.synchronize()
    return out


def oracle_rows(q, k, v, causal, kv_len, scale, dtype, rows=None):
    kind = "bf16" if dtype == "bf16" else "f32"
    kl = None if kv_len is None else kv_len.cpu().numpy()
    return oracle.attention_fp64(oracle_view(q), oracle_view(k), oracle_view(v), scale, causal, kl,
                                 kind=kind, rows=rows)


def gpu_rows(out, rows=None):
    d = out.shape[-1]
    if rows is None:
        return out.float().cpu().numpy().astype(np.float64)
    idx = torch.as_tensor(rows, device=out.device, dtype=torch.long)
    return out.reshape(-1, d).index_select(0, idx).float().cpu().numpy().astype(np.float64)


def compare(got, want, dtype, label=""):
    """Assert the tolerances; return (max_err, mean_err)."""
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{label}: non-finite values in the GPU output"
    err = np.abs(got - want)
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    tmax, tmean = TOL[dtype]
    where = np.unravel_index(int(err.argmax()), err.shape) if err.size else None
    msg = f"{label}: max_err={mx:.3e} (tol {tmax}) mean_err={mean:.3e} (tol {tmean}) worst at {where}"
    assert mx <= tmax, msg
    if tmean is not None:
        assert mean <= tmean, msg
    return mx, mean
