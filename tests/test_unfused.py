"""GPU parity of the operator-centric (unfused) bf16 forward, attn_fwd_unfused,
against the fp64 oracle, through the C ABI.

Same tolerance as the fused bf16 forward (max |err| <= 2e-2, mean |err| <= 2e-3):
the scores are kept in fp32, the probabilities are normalised in fp32 and
rounded to bf16 once, and P V accumulates in fp32, so every step is at least
as precise as in the fused kernel.
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
TOL_MAX, TOL_MEAN = 2e-2, 2e-3


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(got, want, label):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want)
    mx, mn = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    assert mx <= TOL_MAX and mn <= TOL_MEAN, f"{label}: max_err={mx:.3e} mean_err={mn:.3e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_unfused_small_sweep(d, causal, padded):
    # N = 1, 65 and 130 take the scalar paths (N % 4 != 0); 300 and 1000 the
    # vector paths; 130 and 300 leave ragged 128-row tiles
    for N in (1, 65, 130, 300, 1000):
        seed = 1300 + N + 3 * d + 7 * causal + 11 * padded
        q, k, v, kv = make_inputs(2, 3, N, d, "bf16", seed, padded=padded, kv_lo=0 if padded else None)
        scale = float(np.float32(1.0 / math.sqrt(d)))
        _log(f"unfused sweep d={d} causal={causal} padded={padded} N={N} seed={seed}")
        kvd = None if kv is None else kv.to(DEV)
        o = attnio.attn_fwd_unfused(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, kv_len=kvd,
                                    scale=scale, heads_per_pass=2)
        torch.cuda.synchronize()
        want = oracle.attention_fp64(oracle_view(q), oracle_view(k), oracle_view(v), scale, causal,
                                     None if kv is None else kv.numpy(), kind="bf16")
        _check(o.float().cpu().numpy(), want, f"N={N}")


def test_unfused_passes_do_not_change_the_result():
    # one head per pass, several heads per pass and all heads in one pass give
    # bitwise the same output
    q, k, v, kv = make_inputs(3, 2, 257, 128, "bf16", 1401, padded=True, kv_lo=0)
    qd, kd, vd, kvd = q.to(DEV), k.to(DEV), v.to(DEV), kv.to(DEV)
    outs = [attnio.attn_fwd_unfused(qd, kd, vd, kv_len=kvd, causal=True, heads_per_pass=hp)
            for hp in (1, 4, 6)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_unfused_matches_fused_closely():
    # both paths against each other on a peaked input: the same exact result,
    # different roundings; each is within tolerance of the oracle
    q, k, v, _ = make_inputs(1, 2, 700, 64, "bf16", 1402, q_mul=8.0)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    a = attnio.attn_fwd_unfused(qd, kd, vd, causal=True)
    b = attnio.attn_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    want = oracle.attention_fp64(oracle_view(q), oracle_view(k), oracle_view(v), 0.125, True, None,
                                 kind="bf16")
    _check(a.float().cpu().numpy(), want, "unfused")
    _check(b.float().cpu().numpy(), want, "fused")


def test_unfused_workspace_errors():
    q, k, v, _ = make_inputs(1, 1, 64, 64, "bf16", 1403)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    small = torch.empty(attnio.attn_fwd_unfused_workspace_bytes(64) - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(RuntimeError):
        attnio.attn_fwd_unfused(qd, kd, vd, workspace=small)


def test_unfused_headline_workload_sampled():
    # the causal 32768-row workload, four heads per pass, as the benchmark runs it
    w = WORKLOADS["bf16_causal_h32_n32k_d128"]
    _log("unfused headline: inputs")
    q, k, v, _ = workload_inputs(w)
    o = attnio.attn_fwd_unfused(q.to(DEV), k.to(DEV), v.to(DEV), causal=w.causal, scale=w.scale,
                                heads_per_pass=4)
    torch.cuda.synchronize()
    rows = sample_rows(w.B, w.H, w.N, 1024, seed=w.seed)
    _log(f"unfused headline: oracle on {rows.size} rows")
    want = oracle.attention_fp64(oracle_view(q), oracle_view(k), oracle_view(v), w.scale, w.causal,
                                 None, kind="bf16", rows=rows)
    got = o.reshape(-1, w.d).index_select(0, torch.as_tensor(rows, device=DEV)).float().cpu().numpy()
    _check(got, want, "headline")
