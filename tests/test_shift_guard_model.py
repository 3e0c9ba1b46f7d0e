"""CPU model of the overflow guard in the bf16 forward's fast pass (head size 128).

The kernel takes the exponent shift from the first key tile a row sees and
afterwards moves it lazily.  At d = 128 the row sum of a tile's probabilities
is formed on the matrix core, next to the tile's P x V, so the guard that
decides whether the workgroup must recompute its rows in the safe pass sees
that sum only after the product is already in the fp32 accumulator.  This file
replays that order for one query row in numpy float32:

    for each key tile t (in walk order):
        P    = bf16( exp2( fma(s, c, -m) ) )        # m: first tile's row maximum
        acc += P @ V                                # fp32 accumulator
        rs   = sum(P)                               # fp32 row sum of the same P
        bad |= guard(rs)

and shows that a guard on a non-finite row sum alone misses inputs whose
probabilities are finite (up to 2^128) but whose products with V overflow the
accumulator, while the guard on rs <= 2^64 catches them and never fires on
ordinary inputs.  The model is a reading of the kernel's arithmetic order, not
of the attention definition (that is the oracle's job).
"""

import numpy as np

FLT_MAX = float(np.finfo(np.float32).max)
LOG2E = np.float32(1.4426950408889634)
SAFE_SUM_MAX = np.float32(2.0 ** 64)


def _bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (round to nearest even), returned as float32."""
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    finite = np.isfinite(x)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    out = np.where(finite, rounded, bits.astype(np.uint32)).view(np.float32)
    return out


def fast_pass_row(s_row: np.ndarray, v: np.ndarray, c: np.float32, bn: int, guard):
    """Replay the fast pass for one query row.  s_row: fp32 raw scores of the
    visible keys in walk order; v: [keys, d] values.  Returns (acc, l, bad)."""
    nt = (s_row.size + bn - 1) // bn
    m = None
    acc = np.zeros(v.shape[1], dtype=np.float32)
    l_run = np.float32(0)
    bad = False
    with np.errstate(over="ignore", invalid="ignore"):
        for t in range(nt):
            s = s_row[t * bn:(t + 1) * bn].astype(np.float32)
            if m is None:
                m = np.float32(np.max(s * c))
            x = (s * c - m).astype(np.float32)
            p = _bf16(np.exp2(x, dtype=np.float32))
            acc = (acc + (p[:, None] * v[t * bn:(t + 1) * bn].astype(np.float32)).sum(
                axis=0, dtype=np.float32)).astype(np.float32)
            rs = np.float32(p.sum(dtype=np.float32))
            bad = bad or guard(rs)
            l_run = np.float32(l_run + rs)
            if 65536.0 < rs <= SAFE_SUM_MAX:
                mv = np.float32(np.floor(np.log2(rs)))
                alpha = np.float32(np.exp2(-mv))
                acc = (acc * alpha).astype(np.float32)
                l_run = np.float32(l_run * alpha)
                m = np.float32(m + mv)
    return acc, l_run, bad


def old_guard(rs):
    return not (rs <= FLT_MAX)


def new_guard(rs):
    return not (rs <= SAFE_SUM_MAX)


def spike_input(n_keys=300, spike=130, d=128, spike_score=88.0, spike_v=4.0):
    """The GPU test's input for one row: every key scores 0 except one that
    scores spike_score (scale 1, so c = log2 e); V is 1 except the spike row."""
    s = np.zeros(n_keys, dtype=np.float32)
    s[spike] = np.float32(spike_score)
    v = np.ones((n_keys, d), dtype=np.float32)
    v[spike] = spike_v
    return s, v


def test_old_guard_misses_finite_probability_overflow():
    s, v = spike_input()
    acc, l_run, bad = fast_pass_row(s, v, LOG2E, 128, old_guard)
    # the probability itself is finite in bf16 and fp32, so is the row sum ...
    p_spike = _bf16(np.exp2(np.float32(88.0) * LOG2E, dtype=np.float32))
    with np.errstate(over="ignore"):
        assert np.isfinite(p_spike) and p_spike * np.float32(4.0) == np.inf and np.isfinite(l_run)
    # ... the old guard does not fire, and the accumulator holds infinities
    assert not bad
    assert not np.isfinite(acc).all()


def test_new_guard_catches_finite_probability_overflow():
    s, v = spike_input()
    _, _, bad = fast_pass_row(s, v, LOG2E, 128, new_guard)
    assert bad


def test_new_guard_bound_holds_below_threshold():
    """A tile whose row sum is just at the threshold cannot overflow for
    |V| < 2^63: the accumulator stays finite."""
    s, v = spike_input(spike_score=float(63.0 / LOG2E))
    v[130] = 2.0 ** 62
    acc, _, bad = fast_pass_row(s, v, LOG2E, 128, new_guard)
    assert not bad and np.isfinite(acc).all()


def test_new_guard_quiet_on_peaked_random_rows():
    """Rows of the peaked workload's kind (Q x 8, d = 128, scale 1/sqrt(128)):
    the score spread stays far below 64 in the base-2 domain, so the safe pass
    is never requested and the lazy shift handles them."""
    rng = np.random.default_rng(5)
    d, n = 128, 4096
    c = np.float32(np.float32(1 / np.sqrt(d)) * LOG2E)
    for _ in range(8):
        q = _bf16(8.0 * rng.standard_normal(d).astype(np.float32))
        k = _bf16(rng.standard_normal((n, d)).astype(np.float32))
        v = _bf16(rng.standard_normal((n, d)).astype(np.float32))
        s = (k @ q).astype(np.float32)
        acc, l_run, bad = fast_pass_row(s, v, c, 128, new_guard)
        assert not bad and np.isfinite(acc).all() and l_run > 0
        # and the normalised result is the softmax (loosely: the model's
        # rounding is the kernel's, not the oracle's)
        p = np.exp((s.astype(np.float64) - s.max()) * float(c) * np.log(2.0))
        want = (p @ v.astype(np.float64)) / p.sum()
        assert np.abs(acc / l_run - want).max() < 2e-2
