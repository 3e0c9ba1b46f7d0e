"""Plain fp64 CPU oracle for the two streaming row operators: row softmax and
row LayerNorm.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP library and imports neither torch
nor the package; it takes plain numpy arrays.

"From Attention Graph to FlashAttention - A Memory-Centric Compilation
Approach in AICF" names, as the next candidates for the same memory-centric
treatment, streaming softmax and streaming LayerNorm (its closing outlook).
The pages define neither operator further, so each is written here as its
textbook definition over the last axis of an [R, N] matrix, in fp64:

    softmax:    y_j = exp(s x_j) / sum_k exp(s x_k)
                (a row whose entries are all -inf gives a row of zeros, the
                same convention as an attention row with no visible key);
    LayerNorm:  mu = mean_j x_j,  var = mean_j (x_j - mu)^2  (biased),
                y_j = (x_j - mu) / sqrt(var + eps) * gamma_j + beta_j
                (gamma = 1 and beta = 0 when not given).

The softmax subtracts the row maximum before exponentiating, which leaves the
mathematical result unchanged and keeps fp64 exp from overflowing; the
variance is taken in two passes (mean first, then the mean of squared
deviations), its plain definition.

Pinned by tests/test_oracle_rows.py: brute force with math.exp / math.fsum on
tiny rows, closed forms (constant rows, two-valued rows), invariances (shift
for softmax, affine for LayerNorm), scipy's softmax as a special case, and
planted mistakes that the pins must catch.
"""

from __future__ import annotations

import numpy as np

from .attention import to_fp64

__all__ = ["softmax_rows_fp64", "layernorm_rows_fp64"]


def softmax_rows_fp64(x, scale: float = 1.0, kind: str = "bf16") -> np.ndarray:
    """Row softmax of scale * x over the last axis of an [R, N] array, fp64.

    x: 'bf16' uint16 bit patterns, 'f32' or 'f64' values.  scale is the fp32
    value the kernel receives, widened exactly.  Rows of all -inf give zeros."""
    X = to_fp64(np.asarray(x), kind)
    if X.ndim != 2:
        raise ValueError(f"x must be [R, N], got shape {X.shape}")
    s = float(np.float32(scale))
    Z = s * X
    m = Z.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    with np.errstate(invalid="ignore"):
        E = np.exp(Z - m_safe)
    E = np.where(np.isneginf(Z), 0.0, E)
    l = E.sum(axis=1, keepdims=True)
    return np.where(empty, 0.0, E / np.where(empty, 1.0, l))


def layernorm_rows_fp64(x, gamma=None, beta=None, eps: float = 1e-5, kind: str = "bf16") -> np.ndarray:
    """Row LayerNorm of an [R, N] array over its last axis, fp64.

    gamma, beta: None (1 and 0) or length-N arrays of the same kind as x.  eps
    is the fp32 value the kernel receives, widened exactly."""
    X = to_fp64(np.asarray(x), kind)
    if X.ndim != 2:
        raise ValueError(f"x must be [R, N], got shape {X.shape}")
    N = X.shape[1]
    e = float(np.float32(eps))
    mu = X.mean(axis=1, keepdims=True)
    var = ((X - mu) ** 2).mean(axis=1, keepdims=True)
    Y = (X - mu) / np.sqrt(var + e)
    if gamma is not None:
        g = to_fp64(np.asarray(gamma), kind).reshape(1, N)
        Y = Y * g
    if beta is not None:
        b = to_fp64(np.asarray(beta), kind).reshape(1, N)
        Y = Y + b
    return Y
