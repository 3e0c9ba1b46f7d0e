"""GPU parity of the streaming row operators (stream_softmax, stream_layernorm)
against the fp64 oracle, element by element, through the C ABI.

Tolerances (elementwise; derived from the arithmetic):
  softmax:   |y - ref| <= 2^-8 |ref| + 1e-36.  The output is rounded to bf16
             once (<= 2^-9 relative); exp2 and the fp32 sum and reciprocal add
             a few 2^-24 relative, and the fp32 scaling of x adds
             |scale x| 2^-24, far below the remaining 2^-9.  The absolute term
             only covers results in fp32's subnormal range.
  LayerNorm: |y - ref| <= 2^-8 |ref| + 2e-3 |gamma_j| + 1e-6.  The output is
             rounded to bf16 once; the fp32 mean and variance of up to ~10^5
             elements with a mean several standard deviations from zero are
             good to ~1e-4 of a standard deviation, which gamma scales.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from exact_long_sequence_amd import attnio
from exact_long_sequence_amd.inputs import oracle_view

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rand(shape, seed, sd=1.0, mean=0.0):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return (torch.randn(shape, generator=g, dtype=torch.float32) * sd + mean).to(torch.bfloat16)


def _check_softmax(got, want, label):
    got = got.double().cpu().numpy()
    bad = np.abs(got - want) > 2.0 ** -8 * np.abs(want) + 1e-36
    assert not bad.any(), f"{label}: {int(bad.sum())} elements out of tolerance, first at {np.argwhere(bad)[0]}"


def _check_ln(got, want, gamma, label):
    got = got.double().cpu().numpy()
    g = np.ones(want.shape[1]) if gamma is None else np.abs(gamma.double().cpu().numpy())
    bad = np.abs(got - want) > 2.0 ** -8 * np.abs(want) + 2e-3 * g[None, :] + 1e-6
    assert not bad.any(), f"{label}: {int(bad.sum())} elements out of tolerance, first at {np.argwhere(bad)[0]}"


# N covers: a single element, ragged (scalar path), one partial sweep, every
# register-cached sweep count, the largest cached row and streamed rows; for
# LayerNorm also the one-wave-per-row sizes 512, 2048, 4096 and 8192
SIZES = [1, 7, 8, 512, 1000, 2048, 4096, 4104, 8192, 12288, 30000, 65536, 65544, 70001]


@pytest.mark.parametrize("N", SIZES)
def test_softmax_rows(N):
    R = 5
    x = _rand((R, N), 2000 + N, sd=2.0)
    x[1, : max(1, N // 3)] = float("-inf")          # masked entries
    x[2, :] = float("-inf")                          # a fully masked row
    if N > 1:
        x[3, N // 2] = 30.0                          # a dominant entry
    _log(f"softmax R={R} N={N} cached={attnio.stream_rows_cached(N)}")
    xd = x.to(DEV)
    y = attnio.stream_softmax(xd, 0.75)
    torch.cuda.synchronize()
    want = oracle.softmax_rows_fp64(oracle_view(x), 0.75)
    _check_softmax(y, want, f"N={N}")
    assert torch.count_nonzero(y[2]).item() == 0
    # in place gives bitwise the same result
    z = xd.clone()
    attnio.stream_softmax(z, 0.75, out=z)
    torch.cuda.synchronize()
    assert torch.equal(z.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("N", SIZES)
@pytest.mark.parametrize("affine", [False, True])
def test_layernorm_rows(N, affine):
    R = 4
    x = _rand((R, N), 3000 + N, sd=2.0, mean=0.0)
    x[1] = _rand((N,), 3100 + N, sd=0.5, mean=40.0)     # mean far from zero
    x[2] = 1.5                                           # constant row -> beta
    gamma = _rand((N,), 3200 + N, sd=1.0, mean=1.0) if affine else None
    beta = _rand((N,), 3300 + N, sd=0.5) if affine else None
    _log(f"layernorm R={R} N={N} affine={affine} cached={attnio.stream_rows_cached(N)}")
    y = attnio.stream_layernorm(x.to(DEV), None if gamma is None else gamma.to(DEV),
                                None if beta is None else beta.to(DEV), eps=1e-5)
    torch.cuda.synchronize()
    want = oracle.layernorm_rows_fp64(oracle_view(x), None if gamma is None else oracle_view(gamma),
                                      None if beta is None else oracle_view(beta), eps=1e-5)
    _check_ln(y, want, gamma, f"N={N}")


@pytest.mark.parametrize("which", ["gamma", "beta"])
def test_layernorm_one_affine_vector(which):
    # only one of gamma and beta given: the workgroup-per-row kernel at a size
    # that would otherwise take one wave per row
    R, N = 9, 4096
    x = _rand((R, N), 3400, sd=2.0, mean=1.0)
    vec = _rand((N,), 3401, sd=1.0, mean=1.0)
    gamma, beta = (vec, None) if which == "gamma" else (None, vec)
    _log(f"layernorm R={R} N={N} only {which}")
    y = attnio.stream_layernorm(x.to(DEV), None if gamma is None else gamma.to(DEV),
                                None if beta is None else beta.to(DEV), eps=1e-5)
    torch.cuda.synchronize()
    want = oracle.layernorm_rows_fp64(oracle_view(x), None if gamma is None else oracle_view(gamma),
                                      None if beta is None else oracle_view(beta), eps=1e-5)
    _check_ln(y, want, gamma, f"only {which}")


def test_rows_errors_from_binding():
    x = torch.zeros((2, 16), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError):
        attnio.stream_softmax(x, 0.0)
    with pytest.raises(RuntimeError):
        attnio.stream_layernorm(x, eps=-1.0)
    with pytest.raises(ValueError):
        attnio.stream_layernorm(x, gamma=torch.ones(15, dtype=torch.bfloat16, device=DEV))


# the two measured workloads at full size, sampled rows checked one by one
FULL = {
    "softmax_r32k_n32k": (32768, 32768),
    "layernorm_r128k_n8k": (131072, 8192),
}


@pytest.mark.parametrize("name", list(FULL))
def test_rows_full_size_sampled(name):
    from exact_long_sequence_amd.inputs import ROW_WORKLOADS, row_workload_inputs
    w = ROW_WORKLOADS[name]
    assert (w.R, w.N) == FULL[name]
    x, gamma, beta = row_workload_inputs(w)
    _log(f"rows full {name}: GPU")
    xd = x.to(DEV)
    if w.op == "softmax":
        y = attnio.stream_softmax(xd, w.param)
    else:
        y = attnio.stream_layernorm(xd, gamma.to(DEV), beta.to(DEV), eps=w.param)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    rows = np.unique(np.concatenate([rng.choice(w.R, 64, replace=False), [0, w.R - 1]]))
    idx = torch.as_tensor(rows, device=DEV)
    got = y.index_select(0, idx)
    xs = oracle_view(x[torch.as_tensor(rows)])
    _log(f"rows full {name}: oracle on {rows.size} rows")
    if w.op == "softmax":
        _check_softmax(got, oracle.softmax_rows_fp64(xs, w.param), name)
    else:
        _check_ln(got, oracle.layernorm_rows_fp64(xs, oracle_view(gamma), oracle_view(beta), eps=w.param),
                  gamma, name)
