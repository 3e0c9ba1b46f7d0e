"""Pins of the row softmax / LayerNorm oracle (oracle/rows.py) against things
other than itself: brute force in pure Python on tiny rows, closed forms,
invariances, scipy's softmax, and planted mistakes that must be caught."""

import math

import numpy as np
import pytest

import oracle
import oracle.rows as orows


def _brute_softmax(row, s):
    z = [s * v for v in row]
    if all(v == -math.inf for v in z):
        return [0.0] * len(z)
    e = [0.0 if v == -math.inf else math.exp(v) for v in z]   # no max shift: tiny values only
    tot = math.fsum(e)
    return [v / tot for v in e]


def _brute_layernorm(row, g, b, eps):
    n = len(row)
    mu = math.fsum(row) / n
    var = math.fsum((v - mu) ** 2 for v in row) / n
    return [(v - mu) / math.sqrt(var + eps) * g[j] + b[j] for j, v in enumerate(row)]


@pytest.mark.parametrize("N", [1, 2, 5, 17])
def test_softmax_brute_force(N):
    rng = np.random.default_rng(N)
    x = rng.normal(size=(4, N)) * 2
    x[1, 0] = -np.inf
    if N > 1:
        x[2, :] = -np.inf
        x[2, N // 2] = 0.3
    got = oracle.softmax_rows_fp64(x, 0.75, kind="f64")
    for r in range(4):
        np.testing.assert_allclose(got[r], _brute_softmax(list(x[r]), 0.75), rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("N", [1, 2, 5, 17])
def test_layernorm_brute_force(N):
    rng = np.random.default_rng(100 + N)
    x = rng.normal(size=(3, N)) * 3 + 1
    g = rng.normal(size=N)
    b = rng.normal(size=N)
    got = oracle.layernorm_rows_fp64(x, g, b, eps=1e-3, kind="f64")
    e = float(np.float32(1e-3))
    for r in range(3):
        np.testing.assert_allclose(got[r], _brute_layernorm(list(x[r]), g, b, e), rtol=1e-12, atol=1e-12)


def test_softmax_closed_forms():
    # constant row -> uniform; two values a, b -> logistic of s (a - b)
    x = np.full((2, 7), 3.5)
    np.testing.assert_allclose(oracle.softmax_rows_fp64(x, 1.0, kind="f64"), 1 / 7, rtol=1e-15)
    y = oracle.softmax_rows_fp64(np.array([[2.0, -1.0]]), 0.5, kind="f64")
    np.testing.assert_allclose(y[0, 0], 1 / (1 + math.exp(-0.5 * 3.0)), rtol=1e-15)
    # all -inf -> zeros; one finite entry among -inf -> one-hot
    z = np.array([[-np.inf, -np.inf, -np.inf], [-np.inf, 4.0, -np.inf]])
    np.testing.assert_array_equal(oracle.softmax_rows_fp64(z, 1.0, kind="f64"), [[0, 0, 0], [0, 1, 0]])


def test_softmax_shift_invariance_and_scipy():
    special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(7)
    x = rng.normal(size=(5, 300)) * 4
    y = oracle.softmax_rows_fp64(x, 1.25, kind="f64")
    np.testing.assert_allclose(y, oracle.softmax_rows_fp64(x + 123.0, 1.25, kind="f64"), rtol=1e-11)
    np.testing.assert_allclose(y, special.softmax(float(np.float32(1.25)) * x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=1e-14)
    # large entries do not overflow
    big = oracle.softmax_rows_fp64(np.array([[1000.0, 999.0]]), 1.0, kind="f64")
    np.testing.assert_allclose(big[0, 0], 1 / (1 + math.exp(-1)), rtol=1e-14)


def test_layernorm_closed_forms_and_invariance():
    # constant row -> beta exactly (zero deviations)
    x = np.full((1, 9), -2.5)
    b = np.arange(9.0)
    np.testing.assert_array_equal(oracle.layernorm_rows_fp64(x, None, b, 1e-5, kind="f64"), b[None])
    # two values +-a: normalised to +-a / sqrt(a^2 + eps)
    a, e = 3.0, float(np.float32(1e-5))
    y = oracle.layernorm_rows_fp64(np.array([[a, -a, a, -a]]) + 10, None, None, 1e-5, kind="f64")
    np.testing.assert_allclose(y, [[a / math.sqrt(a * a + e), -a / math.sqrt(a * a + e)] * 2], rtol=1e-14)
    # without affine terms: mean 0, variance var/(var+eps); affine invariance in x
    rng = np.random.default_rng(9)
    x = rng.normal(size=(4, 500)) * 2 + 5
    y0 = oracle.layernorm_rows_fp64(x, None, None, 0.0, kind="f64")
    np.testing.assert_allclose(y0.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((y0 ** 2).mean(axis=1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(oracle.layernorm_rows_fp64(3 * x - 7, None, None, 0.0, kind="f64"), y0, atol=1e-12)


def test_bf16_inputs_are_widened_exactly():
    bits = np.array([[0x3F80, 0x4000, 0xC040]], dtype=np.uint16)      # 1, 2, -3
    np.testing.assert_allclose(oracle.softmax_rows_fp64(bits, 1.0), [_brute_softmax([1.0, 2.0, -3.0], 1.0)],
                               rtol=1e-14)
    np.testing.assert_allclose(oracle.layernorm_rows_fp64(bits, None, None, 0.0),
                               [_brute_layernorm([1.0, 2.0, -3.0], [1] * 3, [0] * 3, 0.0)], rtol=1e-14)


def test_planted_mistakes_are_caught(monkeypatch):
    """Each plausible slip in the oracle, planted on the CPU, fails a pin."""
    rng = np.random.default_rng(11)
    x = rng.normal(size=(3, 6))
    g, b = rng.normal(size=6), rng.normal(size=6)
    want_s = [_brute_softmax(list(r), 0.9) for r in x]
    e = float(np.float32(1e-2))
    want_l = [_brute_layernorm(list(r), g, b, e) for r in x]

    def mutants():
        def unbiased(X, gamma=None, beta=None, eps=1e-5, kind="f64"):   # N-1 variance
            X = np.asarray(X, float); mu = X.mean(1, keepdims=True)
            v = ((X - mu) ** 2).sum(1, keepdims=True) / (X.shape[1] - 1)
            return (X - mu) / np.sqrt(v + eps) * gamma + beta
        def eps_outside(X, gamma=None, beta=None, eps=1e-5, kind="f64"):  # sqrt(var) + eps
            X = np.asarray(X, float); mu = X.mean(1, keepdims=True)
            v = ((X - mu) ** 2).mean(1, keepdims=True)
            return (X - mu) / (np.sqrt(v) + eps) * gamma + beta
        def no_scale(X, scale=1.0, kind="f64"):
            return orows.softmax_rows_fp64(X, 1.0, kind)
        def col_norm(X, scale=1.0, kind="f64"):                           # normalised the wrong axis
            Z = np.exp(float(np.float32(scale)) * np.asarray(X, float))
            return Z / Z.sum(0, keepdims=True)
        return [("layernorm", unbiased), ("layernorm", eps_outside), ("softmax", no_scale),
                ("softmax", col_norm)]

    for kind, fn in mutants():
        if kind == "softmax":
            got = fn(x, 0.9, kind="f64")
            assert not np.allclose(got, want_s, rtol=1e-12), fn.__name__
        else:
            got = fn(x, g, b, e, kind="f64")
            assert not np.allclose(got, want_l, rtol=1e-12), fn.__name__
