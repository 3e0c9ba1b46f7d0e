"""The allocation-free backward entry point, attn_bwd_noalloc, through the C ABI.

It runs the same kernels as attn_bwd with the row statistics in the library's
static device scratch instead of a caller workspace, so its gradients must be
bitwise those of attn_bwd on the same inputs (and so within the backward's
tolerance of the oracle).  Two calls in a row, the second on a smaller input,
check that the shared scratch carries nothing from one call into the next;
a shape whose statistics exceed the scratch is refused before any launch.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from exact_long_sequence_amd import attnio
from exact_long_sequence_amd.inputs import make_inputs, oracle_view

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _case(B, H, N, d, causal, padded, seed):
    q, k, v, kv = make_inputs(B, H, N, d, "bf16", seed=seed, padded=padded, kv_lo=1)
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    return q, k, v, kv, do


def _grads(fn, qd, kd, vd, o, dod, lse, causal, kvd, **kw):
    dq, dk, dv = (torch.full_like(qd, float("nan")) for _ in range(3))
    fn(qd, kd, vd, o, dod, lse, causal=causal, kv_len=kvd, dq=dq, dk=dk, dv=dv, **kw)
    torch.cuda.synchronize()
    return dq, dk, dv


def test_noalloc_matches_workspace_backward_two_calls():
    cases = [(2, 3, 700, 128, True, True, 51), (1, 2, 300, 64, False, False, 52)]
    for (B, H, N, d, causal, padded, seed) in cases:   # the second input is smaller
        print(f"noalloc case B={B} H={H} N={N} d={d} causal={causal} padded={padded}", flush=True)
        sys.stdout.flush()
        q, k, v, kv, do = _case(B, H, N, d, causal, padded, seed)
        qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
        kvd = None if kv is None else kv.to(DEV)
        o, lse = attnio.attn_fwd_lse(qd, kd, vd, causal=causal, kv_len=kvd)
        ws = torch.full((attnio.attn_bwd_workspace_bytes(B, H, N),), 0xFF, dtype=torch.uint8, device=DEV)
        ref = _grads(attnio.attn_bwd, qd, kd, vd, o, dod, lse, causal, kvd, workspace=ws)
        got = _grads(attnio.attn_bwd_noalloc, qd, kd, vd, o, dod, lse, causal, kvd)
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.isfinite(a.float()).all(), name
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
        # and against the oracle, to the backward's tolerance
        refs = oracle.attention_bwd_fp64(oracle_view(q), oracle_view(k), oracle_view(v), oracle_view(do),
                                         float(np.float32(1 / np.sqrt(d))), causal,
                                         None if kv is None else kv.numpy(), kind="bf16")
        for name, t, r in zip(("dQ", "dK", "dV"), got, refs):
            e = np.abs(t.float().cpu().numpy().astype(np.float64) - r)
            assert e.max() <= 2.5e-2 * np.abs(r).max() + 1e-6, name
            assert e.mean() <= 1e-2 * np.abs(r).mean() + 1e-7, name


def test_noalloc_refuses_shapes_beyond_its_scratch():
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(1, 1, 64, dtype=torch.float32, device=DEV)
    lib = attnio.load_library()
    # B*H*NP rows of 8 bytes: 4194304 rows fit the 32 MiB scratch, one more 64-row block does not
    B, H, N = 1, 4097, 1024
    assert attnio.attn_bwd_workspace_bytes(B, H, N) > 32 * 1024 * 1024
    outs = [torch.empty(1, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    # host-side refusal: pointers are never dereferenced for a refused shape
    rc = lib.attn_bwd_noalloc(x.data_ptr(), x.data_ptr() + (1 << 30), x.data_ptr() + (2 << 30),
                              x.data_ptr() + (3 << 30), x.data_ptr() + (4 << 30), lse.data_ptr() + (5 << 30),
                              x.data_ptr() + (6 << 30), x.data_ptr() + (7 << 30), x.data_ptr() + (8 << 30),
                              B, H, N, 64, 0.125, 0, None, None)
    assert rc == -9, rc
    del outs
