"""GPU parity of the fp8 (OCP E4M3) attention forward, attn_fwd_fp8, against the
fp64 oracle of the same fp8 inputs, through the C ABI.

The oracle decodes the E4M3 bytes exactly and applies the descales, so input
quantisation is not part of the error; what remains is the kernel's own
rounding.  Tolerance, elementwise, derived from it:
    |O - O_ref| <= (M + |O_ref|) / 15 + 2^-9 |O_ref| + 2e-3,   M = |P| |V| (oracle),
    mean |O - O_ref| <= 2^-6 mean(M).
Each probability is rounded to E4M3 once, p_j (1 + d_j) with |d_j| <= 2^-4 in
the format's normal range, and the row sum is the sum of those same rounded
values, so O = sum_j P_j (1 + d_j) V_j / (1 + db) with db = sum_j P_j d_j:
O - O_ref = (sum_j P_j d_j V_j - db O_ref) / (1 + db), at most
2^-4 (M + |O_ref|) / (1 - 2^-4) = (M + |O_ref|) / 15; the output's bf16
rounding adds 2^-9 |O|.  Probabilities in E4M3's subnormal range (below 2^-6,
that is 2^-14 to 2^-14.75 of the row's largest probability, which the kernel
keeps in [2^8, 2^8.75 = 430.5] by letting its exponent shift trail the running
maximum by up to 0.75) round with an absolute error of at most 2^-10, at most
2^-18 of the largest probability each; with the fp32
accumulation they stay far inside the 2e-3 term (a CPU model of exactly these
roundings, per-tile shifts included, exceeds the first two terms by at most
5e-6 on the shapes below, reaches at most 0.59 of the bound, and its mean
error is at most 0.63% of mean(M)).
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_long_sequence_amd import attnio
from exact_long_sequence_amd.inputs import make_fp8_inputs, sample_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(got, want, mag, label):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    err = np.abs(got - want)
    bound = (mag + np.abs(want)) / 15.0 + 2.0 ** -9 * np.abs(want) + 2e-3
    bad = err > bound
    ratio = float(np.max(err / bound)) if err.size else 0.0
    mean_ok = err.mean() <= 2.0 ** -6 * mag.mean() + 1e-12 if err.size else True
    _log(f"  {label}: max err {err.max(initial=0):.3e}, max err/bound {ratio:.3f}, "
         f"mean err {err.mean() if err.size else 0:.3e}, mean M {mag.mean() if mag.size else 0:.3e}")
    assert not bad.any(), f"{label}: {int(bad.sum())} elements out of tolerance (max err/bound {ratio:.3f})"
    assert mean_ok, f"{label}: mean error {err.mean():.3e} above 2^-6 mean(M)"


def _bits(t):
    return t.numpy()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_fp8_small_sweep(d, causal, padded):
    for N in (1, 65, 300, 1000):
        for q_mul in (1.0, 8.0):
            seed = 4000 + N + 3 * d + 7 * causal + 11 * padded + int(q_mul)
            q8, k8, v8, ds, kv = make_fp8_inputs(2, 2, N, d, seed, padded=padded, q_mul=q_mul,
                                                 kv_lo=0 if padded else None)
            scale = float(np.float32(1.0 / math.sqrt(d)))
            _log(f"fp8 sweep d={d} causal={causal} padded={padded} N={N} q_mul={q_mul} seed={seed} "
                 f"descale={ds}")
            kvd = None if kv is None else kv.to(DEV)
            o = attnio.attn_fwd_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), ds, causal=causal, kv_len=kvd,
                                    scale=scale)
            torch.cuda.synchronize()
            want, mag = oracle.attention_fp8_fp64(_bits(q8), _bits(k8), _bits(v8), ds, scale, causal,
                                                  None if kv is None else kv.numpy(), magnitude=True)
            _check(o.float().cpu().numpy(), want, mag, f"N={N} q_mul={q_mul}")
            if kv is not None:
                for b in range(2):
                    if int(kv[b]) == 0:
                        assert torch.count_nonzero(o[b]).item() == 0


def test_fp8_descales_and_errors():
    # scaling a descale by 2 scales the output exactly (v) or changes only the
    # softmax temperature (q, k): compare against the oracle with the same descales
    q8, k8, v8, ds, _ = make_fp8_inputs(1, 2, 200, 128, 4100)
    qd, kd, vd = q8.to(DEV), k8.to(DEV), v8.to(DEV)
    o1 = attnio.attn_fwd_fp8(qd, kd, vd, ds)
    o2 = attnio.attn_fwd_fp8(qd, kd, vd, (ds[0], ds[1], ds[2] * 2))
    torch.cuda.synchronize()
    assert torch.equal((o1.float() * 2).to(torch.bfloat16).view(torch.int16), o2.view(torch.int16))
    ds2 = (ds[0] * 4, ds[1], ds[2])
    o3 = attnio.attn_fwd_fp8(qd, kd, vd, ds2)
    torch.cuda.synchronize()
    want, mag = oracle.attention_fp8_fp64(_bits(q8), _bits(k8), _bits(v8), ds2, 1 / math.sqrt(128), False,
                                          None, magnitude=True)
    _check(o3.float().cpu().numpy(), want, mag, "q descale x4")
    with pytest.raises(RuntimeError):
        attnio.attn_fwd_fp8(qd, kd, vd, (0.0, 1.0, 1.0))
    with pytest.raises(TypeError):
        attnio.attn_fwd_fp8(qd.to(torch.int8), kd, vd, ds)


def test_fp8_headline_workload_sampled():
    # the causal 32768-row, 32-head, d = 128 shape with fp8 inputs
    B, H, N, d = 1, 32, 32768, 128
    _log("fp8 headline: inputs")
    q8, k8, v8, ds, _ = make_fp8_inputs(B, H, N, d, 1003)
    o = attnio.attn_fwd_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), ds, causal=True)
    torch.cuda.synchronize()
    rows = sample_rows(B, H, N, 1024, seed=1003)
    _log(f"fp8 headline: oracle on {rows.size} rows")
    want, mag = oracle.attention_fp8_fp64(_bits(q8), _bits(k8), _bits(v8), ds, 1 / math.sqrt(d), True, None,
                                          rows=rows, magnitude=True)
    got = o.reshape(-1, d).index_select(0, torch.as_tensor(rows, device=DEV)).float().cpu().numpy()
    _check(got, want, mag, "headline")


@pytest.mark.parametrize("scale", [0.0, -0.07])
def test_fp8_zero_and_negative_scale(scale):
    # scale 0 gives uniform weights over the visible keys; a negative scale
    # favours the smallest scores; masking must hold in both
    q8, k8, v8, ds, kv = make_fp8_inputs(2, 2, 300, 64, 4200, padded=True, kv_lo=0)
    o = attnio.attn_fwd_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), ds, causal=True, kv_len=kv.to(DEV),
                            scale=scale)
    torch.cuda.synchronize()
    want, mag = oracle.attention_fp8_fp64(_bits(q8), _bits(k8), _bits(v8), ds, scale, True, kv.numpy(),
                                          magnitude=True)
    _check(o.float().cpu().numpy(), want, mag, f"scale={scale}")
