"""Pins for the fp64 oracle (CPU only).

The pages print no worked numeric example, so every pin is one of: brute force
on tiny inputs (a pure-Python loop written independently of the oracle, without
the max shift and without numpy), a closed form, an invariant of the definition,
or a library routine (scipy's softmax).  Each is chosen so that a plausible
mistake in the oracle (a dropped scale, a strict causal compare, a transposed
operand, padding ignored, missing normalisation, a wrong bf16 widening) fails
at least one of them; test_mutants_are_caught plants such mistakes on the CPU
and checks that they are caught.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.attention as oa


# --------------------------------------------------------------------------
# brute force: the operator graph (scores, mask, softmax, weighted sum) with
# Python floats, math.exp and math.fsum, one query row at a time
# --------------------------------------------------------------------------
def brute_force(q, k, v, scale, causal, kv_len):
    B, H, N, d = q.shape
    out = np.zeros((B, H, N, d))
    s = float(np.float32(scale))
    for b in range(B):
        L = N if kv_len is None else max(0, min(int(kv_len[b]), N))
        for h in range(H):
            for i in range(N):
                keys = [j for j in range(N) if j < L and (not causal or j <= i)]
                if not keys:
                    continue
                w = {}
                for j in keys:
                    dot = math.fsum(float(q[b, h, i, t]) * float(k[b, h, j, t]) for t in range(d))
                    w[j] = math.exp(s * dot)
                Z = math.fsum(w.values())
                for t in range(d):
                    out[b, h, i, t] = math.fsum(w[j] * float(v[b, h, j, t]) for j in keys) / Z
    return out


def _rand(shape, seed, sd=0.7):
    return np.random.default_rng(seed).normal(0.0, sd, size=shape)


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("d", [1, 2, 4, 8])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_brute_force_tiny(N, d, causal, padded):
    seed = 100 * N + 10 * d + 2 * causal + padded
    B, H = 2, 2
    q, k, v = (_rand((B, H, N, d), seed + t) for t in range(3))
    kv_len = None
    if padded:
        kv_len = np.random.default_rng(seed + 7).integers(0, N + 1, size=B)
    scale = 1.0 / math.sqrt(d)
    got = oracle.attention_fp64(q, k, v, scale, causal, kv_len, kind="f64")
    ref = brute_force(q, k, v, scale, causal, kv_len)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_brute_force_bf16_bits():
    """bf16 path: bit patterns from torch's round-to-nearest-even conversion."""
    torch = pytest.importorskip("torch")
    g = torch.Generator().manual_seed(5)
    B, H, N, d = 1, 2, 7, 4
    t = [torch.randn(B, H, N, d, generator=g).to(torch.bfloat16) for _ in range(3)]
    bits = [x.view(torch.int16).numpy().view(np.uint16) for x in t]
    vals = [x.to(torch.float64).numpy() for x in t]
    kv = np.array([5])
    got = oracle.attention_fp64(*bits, 0.5, True, kv, kind="bf16")
    ref = brute_force(*vals, 0.5, True, kv)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# bf16 widening
# --------------------------------------------------------------------------
def test_bf16_decoder_known_patterns():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4000, 0xC040, 0x3F00, 0x7F80, 0xFF80,
                     0x0001, 0x7F7F, 0x3E80], dtype=np.uint16)
    want = [0.0, -0.0, 1.0, -1.0, 2.0, -3.0, 0.5, np.inf, -np.inf,
            2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, 0.25]
    got = oa.decode_bf16_bits(bits)
    for g_, w_ in zip(got, want):
        assert g_ == w_ and math.copysign(1, g_) == math.copysign(1, w_)
    assert np.isnan(oracle.decode_bf16_bits(np.array([0x7FC0], dtype=np.uint16))[0])


def test_bf16_decoder_matches_torch():
    torch = pytest.importorskip("torch")
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    tb = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = oracle.decode_bf16_bits(allbits)
    same = (ours == tb) | (np.isnan(ours) & np.isnan(tb))
    assert same.all()


def test_bf16_decoder_rejects_other_dtypes():
    with pytest.raises(TypeError):
        oracle.decode_bf16_bits(np.zeros(3, dtype=np.int32))


# --------------------------------------------------------------------------
# invariants and closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows(causal):
    B, H, N, d = 2, 3, 33, 8
    q, k, v = (_rand((B, H, N, d), 11 + t, 1.5) for t in range(3))
    kv = np.array([20, 33])
    O, P, lse = oracle.attention_full_fp64(q, k, v, 0.35, causal, kv)
    assert (P >= 0).all()
    for b in range(B):
        L = kv[b]
        i = np.arange(N)[:, None]
        j = np.arange(N)[None, :]
        allowed = np.broadcast_to((j < L) & ((j <= i) if causal else True), (N, N))
        assert (P[b][:, ~allowed] == 0).all()   # masked entries are exactly zero
        np.testing.assert_allclose(P[b].sum(-1), 1.0, rtol=0, atol=1e-12)
        # lse is log sum exp of the allowed scaled scores
        S = float(np.float32(0.35)) * np.einsum("hid,hjd->hij", q[b], k[b])
        S = np.where(allowed, S, -np.inf)
        ref = np.log(np.exp(S).sum(-1))
        np.testing.assert_allclose(lse[b], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_that_constant(causal):
    B, H, N, d = 1, 2, 50, 16
    q, k = _rand((B, H, N, d), 1, 2.0), _rand((B, H, N, d), 2, 2.0)
    c = _rand((d,), 3)
    v = np.broadcast_to(c, (B, H, N, d)).copy()
    O = oracle.attention_fp64(q, k, v, 0.25, causal, np.array([37]), kind="f64")
    np.testing.assert_allclose(O, np.broadcast_to(c, O.shape), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_is_uniform_mean(causal):
    B, H, N, d = 2, 1, 40, 8
    q, k, v = (_rand((B, H, N, d), 20 + t) for t in range(3))
    kv = np.array([40, 13])
    O = oracle.attention_fp64(q, k, v, 0.0, causal, kv, kind="f64")
    for b in range(B):
        L = kv[b]
        for i in range(N):
            n = min(i + 1, L) if causal else L
            want = v[b, 0, :n].mean(0)
            np.testing.assert_allclose(O[b, 0, i], want, rtol=0, atol=1e-12)


def test_zero_scale_causal_prefix_mean_cumsum():
    N, d = 300, 4
    v = _rand((1, 1, N, d), 30)
    q = k = _rand((1, 1, N, d), 31)
    O = oracle.attention_fp64(q, k, v, 0.0, True, None, kind="f64")
    want = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(O[0, 0], want, rtol=0, atol=1e-12)


def test_causal_first_row_and_single_key():
    B, H, N, d = 1, 2, 9, 8
    q, k, v = (_rand((B, H, N, d), 40 + t, 3.0) for t in range(3))
    O = oracle.attention_fp64(q, k, v, 0.9, True, None, kind="f64")
    np.testing.assert_array_equal(O[:, :, 0], v[:, :, 0])         # row 0 sees key 0 only
    O1 = oracle.attention_fp64(q[:, :, :1], k[:, :, :1], v[:, :, :1], 0.9, False, None, kind="f64")
    np.testing.assert_array_equal(O1, v[:, :, :1])                 # N = 1: O = V
    O2 = oracle.attention_fp64(q, k, v, 0.9, False, np.array([1]), kind="f64")
    np.testing.assert_array_equal(O2, np.broadcast_to(v[:, :, :1], O2.shape))  # kv_len = 1


def test_fully_masked_rows_are_zero():
    q, k, v = (_rand((2, 1, 6, 4), 50 + t) for t in range(3))
    O = oracle.attention_fp64(q, k, v, 0.5, False, np.array([0, 6]), kind="f64")
    assert (O[0] == 0).all() and np.isfinite(O).all()
    O = oracle.attention_fp64(q, k, v, 0.5, True, np.array([0, -3]), kind="f64")  # clamped to 0
    assert (O == 0).all()


def test_kv_len_clamped_above():
    q, k, v = (_rand((1, 1, 6, 4), 55 + t) for t in range(3))
    a = oracle.attention_fp64(q, k, v, 0.5, False, np.array([600]), kind="f64")
    b = oracle.attention_fp64(q, k, v, 0.5, False, None, kind="f64")
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_masked_keys_contribute_nothing(causal):
    B, H, N, d = 1, 2, 64, 16
    q, k, v = (_rand((B, H, N, d), 60 + t) for t in range(3))
    L = 41
    k2, v2 = k.copy(), v.copy()
    k2[:, :, L:] = _rand((B, H, N - L, d), 70, 50.0)
    v2[:, :, L:] = _rand((B, H, N - L, d), 71, 50.0)
    a = oracle.attention_fp64(q, k, v, 0.3, causal, np.array([L]), kind="f64")
    b = oracle.attention_fp64(q, k2, v2, 0.3, causal, np.array([L]), kind="f64")
    np.testing.assert_array_equal(a, b)
    if causal:
        # the future of row i never matters: perturbing keys > i leaves row i unchanged
        i = 10
        k3, v3 = k.copy(), v.copy()
        k3[:, :, i + 1:] += 5.0
        v3[:, :, i + 1:] -= 7.0
        c = oracle.attention_fp64(q, k3, v3, 0.3, True, None, kind="f64")
        a2 = oracle.attention_fp64(q, k, v, 0.3, True, None, kind="f64")
        np.testing.assert_array_equal(a2[:, :, : i + 1], c[:, :, : i + 1])


def test_ramp_closed_form():
    """Q_i = u, K_j = t_j u with increasing t_j: the row maximum grows with every
    key, and O_i[0] = sum_j j w_j / sum_j w_j with w_j = exp(s t_j |u|^2)."""
    N, d = 200, 8
    u = _rand((d,), 80)
    u /= np.linalg.norm(u)
    t = np.linspace(-3.0, 9.0, N)
    q = np.broadcast_to(u, (1, 1, N, d)).copy()
    k = (t[:, None] * u[None, :])[None, None]
    v = np.zeros((1, 1, N, d))
    v[0, 0, :, 0] = np.arange(N)
    v[0, 0, :, 1] = 1.0
    s = 1.75
    O = oracle.attention_fp64(q, k, v, s, True, None, kind="f64")
    s64 = float(np.float32(s))
    for i in (0, 1, 57, 128, N - 1):
        w = np.exp(s64 * t[: i + 1] - s64 * t[i])
        want = (np.arange(i + 1) * w).sum() / w.sum()
        assert abs(O[0, 0, i, 0] - want) <= 1e-10 * max(1.0, abs(want))
        assert abs(O[0, 0, i, 1] - 1.0) <= 1e-12


def test_permutation_and_shift_invariance():
    B, H, N, d = 1, 1, 48, 8
    q, k, v = (_rand((B, H, N, d), 90 + t) for t in range(3))
    base = oracle.attention_fp64(q, k, v, 0.4, False, None, kind="f64")
    perm = np.random.default_rng(91).permutation(N)
    # jointly permuting keys and values leaves every row unchanged
    pk = oracle.attention_fp64(q, k[:, :, perm], v[:, :, perm], 0.4, False, None, kind="f64")
    np.testing.assert_allclose(pk, base, rtol=0, atol=1e-12)
    # permuting queries permutes output rows
    pq = oracle.attention_fp64(q[:, :, perm], k, v, 0.4, False, None, kind="f64")
    np.testing.assert_allclose(pq, base[:, :, perm], rtol=0, atol=1e-12)
    # adding one vector to every key adds a per-row constant to the scores
    w = _rand((d,), 92)
    sh = oracle.attention_fp64(q, k + w, v, 0.4, False, None, kind="f64")
    np.testing.assert_allclose(sh, base, rtol=0, atol=1e-12)


def test_matches_scipy_softmax():
    special = pytest.importorskip("scipy.special")
    B, H, N, d = 1, 2, 257, 32
    q, k, v = (_rand((B, H, N, d), 95 + t, 1.2) for t in range(3))
    s = 1 / math.sqrt(d)
    O = oracle.attention_fp64(q, k, v, s, True, None, kind="f64")
    s64 = float(np.float32(s))
    for h in range(H):
        S = s64 * q[0, h] @ k[0, h].T
        S[np.triu_indices(N, 1)] = -np.inf
        want = special.softmax(S, axis=-1) @ v[0, h]
        np.testing.assert_allclose(O[0, h], want, rtol=0, atol=1e-12)


def test_scale_is_the_fp32_value():
    """The oracle uses fp32(scale) widened, not the fp64 number passed in."""
    q, k, v = (_rand((1, 1, 5, 3), 96 + t, 4.0) for t in range(3))
    s = 1 / math.sqrt(128)
    a = oracle.attention_fp64(q, k, v, s, False, None, kind="f64")
    b = oracle.attention_fp64(q, k, v, float(np.float32(s)), False, None, kind="f64")
    np.testing.assert_array_equal(a, b)


def test_row_selection_matches_full_output():
    B, H, N, d = 2, 3, 70, 8
    q, k, v = (_rand((B, H, N, d), 100 + t) for t in range(3))
    kv = np.array([70, 31])
    full = oracle.attention_fp64(q, k, v, 0.3, True, kv, kind="f64")
    rows = np.random.default_rng(3).choice(B * H * N, 77, replace=False)
    part = oracle.attention_fp64(q, k, v, 0.3, True, kv, kind="f64", rows=rows, chunk=16)
    np.testing.assert_allclose(part, full.reshape(-1, d)[rows], rtol=0, atol=1e-13)


def test_input_validation():
    x = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention_fp64(x, x[:, :, :3], x, 1.0, kind="f64")
    with pytest.raises(ValueError):
        oracle.attention_fp64(x, x, x, 1.0, kind="f64", kv_len=np.array([1, 2]))
    with pytest.raises(ValueError):
        oracle.attention_fp64(x, x, x, 1.0, kind="f64", rows=np.array([4]))
    with pytest.raises(TypeError):
        oracle.attention_fp64(x, x, x, 1.0, kind="f32")


# --------------------------------------------------------------------------
# planted mistakes (on the CPU, in the oracle) must be caught by the pins
# --------------------------------------------------------------------------
def _pins_pass():
    try:
        test_brute_force_tiny(5, 4, True, True)
        test_brute_force_tiny(8, 2, False, True)
        test_probability_rows(True)
        test_masked_keys_contribute_nothing(False)
        test_bf16_decoder_known_patterns()
        test_brute_force_bf16_bits()
        test_causal_first_row_and_single_key()
    except AssertionError:
        return False
    return True


def test_mutants_are_caught(monkeypatch):
    assert _pins_pass()
    real_mask = oa.allowed_mask
    real_soft = oa._softmax_rows
    real_dec = oa.decode_bf16_bits
    mutants = {
        "strict_causal": lambda rows, n, L, c: real_mask(rows, n, L, c) & (
            (np.arange(n)[None, :] < np.asarray(rows)[:, None]) if c else True),
        "padding_ignored": lambda rows, n, L, c: real_mask(rows, n, n, c),
        "off_by_one_padding": lambda rows, n, L, c: real_mask(rows, n, L + 1, c),
    }
    for name, fn in mutants.items():
        monkeypatch.setattr(oa, "allowed_mask", fn)
        assert not _pins_pass(), name
        monkeypatch.setattr(oa, "allowed_mask", real_mask)

    def unnormalised(S, ok):
        P, lse = real_soft(S, ok)
        return P * 1.01, lse
    monkeypatch.setattr(oa, "_softmax_rows", unnormalised)
    assert not _pins_pass()
    monkeypatch.setattr(oa, "_softmax_rows", real_soft)

    monkeypatch.setattr(oa, "decode_bf16_bits",
                        lambda b: (np.asarray(b).astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64))
    assert not _pins_pass()
    monkeypatch.setattr(oa, "decode_bf16_bits", real_dec)

    real_rows = oa.attention_rows_fp64

    def transposed_kv(Qf, Kf, Vf, *a, **kw):
        return real_rows(Qf, Vf, Kf, *a, **kw)
    monkeypatch.setattr(oa, "attention_rows_fp64", transposed_kv)
    assert not _pins_pass()

    def no_scale(Qf, Kf, Vf, rows, scale, *a, **kw):
        return real_rows(Qf, Kf, Vf, rows, 1.0, *a, **kw)
    monkeypatch.setattr(oa, "attention_rows_fp64", no_scale)
    assert not _pins_pass()
    monkeypatch.setattr(oa, "attention_rows_fp64", real_rows)
    assert _pins_pass()


# --------------------------------------------------------------------------
# log-sum-exp side output: brute force with math.exp / math.fsum / math.log
# --------------------------------------------------------------------------
def brute_force_lse(q, k, scale, causal, kv_len):
    B, H, N, d = q.shape
    out = np.full((B, H, N), -np.inf)
    s = float(np.float32(scale))
    for b in range(B):
        L = N if kv_len is None else max(0, min(int(kv_len[b]), N))
        for h in range(H):
            for i in range(N):
                keys = [j for j in range(N) if j < L and (not causal or j <= i)]
                if keys:
                    out[b, h, i] = math.log(math.fsum(
                        math.exp(s * math.fsum(float(q[b, h, i, t]) * float(k[b, h, j, t])
                                               for t in range(d))) for j in keys))
    return out


@pytest.mark.parametrize("N", [1, 3, 8, 13])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_lse_brute_force_tiny(N, causal, padded):
    B, H, d = 2, 2, 4
    seed = 7000 + 10 * N + 2 * causal + padded
    q, k, v = (_rand((B, H, N, d), seed + t) for t in range(3))
    kv_len = np.array([0, N]) if padded else None
    got = oracle.attention_lse_fp64(q, k, v, 0.5, causal, kv_len, kind="f64")
    ref = brute_force_lse(q, k, 0.5, causal, kv_len)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    fin = np.isfinite(ref)
    np.testing.assert_allclose(got[fin], ref[fin], rtol=0, atol=1e-12)
    # rows selected by flat index give the same values
    rows = np.array([0, B * H * N - 1, (B * H * N) // 2])
    np.testing.assert_allclose(
        oracle.attention_lse_fp64(q, k, v, 0.5, causal, kv_len, kind="f64", rows=rows),
        got.reshape(-1)[rows], rtol=0, atol=1e-13)


def test_lse_closed_forms():
    """Zero scale: lse = ln(number of visible keys).  Equal scores c over n keys:
    lse = c + ln n (q = e_0, k_j = (1, ...))."""
    B, H, N, d = 1, 1, 9, 3
    q = _rand((B, H, N, d), 1)
    k = _rand((B, H, N, d), 2)
    lse = oracle.attention_lse_fp64(q, k, k, 0.0, True, None, kind="f64")
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, N + 1)), atol=1e-14)
    q1 = np.zeros((B, H, N, d)); q1[..., 0] = 1.0
    k1 = np.zeros((B, H, N, d)); k1[..., 0] = 2.0
    lse1 = oracle.attention_lse_fp64(q1, k1, k1, 0.75, False, [5], kind="f64")
    np.testing.assert_allclose(lse1[0, 0], 0.75 * 2.0 + np.log(5.0), atol=1e-14)


# --------------------------------------------------------------------------
# backward: central finite differences of the forward oracle (an independent
# check of every gradient formula), plus the zero-gradient rules for masked keys
# --------------------------------------------------------------------------
def _loss(q, k, v, do, scale, causal, kv_len):
    return float((oracle.attention_fp64(q, k, v, scale, causal, kv_len, kind="f64") * do).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_backward_matches_finite_differences(causal, padded):
    B, H, N, d = 2, 1, 6, 3
    seed = 9100 + 2 * causal + padded
    q, k, v, do = (_rand((B, H, N, d), seed + t, sd=0.9) for t in range(4))
    kv_len = np.array([4, 6]) if padded else None
    scale = 0.8
    dq, dk, dv = oracle.attention_bwd_fp64(q, k, v, do, scale, causal, kv_len, kind="f64")
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, scale, causal, kv_len)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, scale, causal, kv_len)
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=0, atol=2e-8, err_msg=f"d{name}")
    if padded:
        assert (dk[0, :, 4:] == 0).all() and (dv[0, :, 4:] == 0).all()


def test_backward_invariants():
    """Each row of dS sums to zero, so dQ is unchanged when every key row of K
    shifts by the same vector; dV sums to sum_i dO_i over rows that see keys."""
    B, H, N, d = 1, 2, 7, 4
    q, k, v, do = (_rand((B, H, N, d), 9300 + t) for t in range(4))
    dq, dk, dv = oracle.attention_bwd_fp64(q, k, v, do, 0.6, True, None, kind="f64")
    shift = np.random.default_rng(5).normal(size=(1, 1, 1, d))
    dq2, _, _ = oracle.attention_bwd_fp64(q, k + shift, v, do, 0.6, True, None, kind="f64")
    np.testing.assert_allclose(dq, dq2, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)   # sum_j dK_j = s sum_i (sum_j dS_ij) q_i = 0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_sampled_backward_matches_finite_differences(causal, padded):
    """The chunked, sampled backward against central differences of the forward
    oracle's loss, with chunks smaller than N so rows and keys span chunks."""
    B, H, N, d = 2, 2, 7, 3
    seed = 9500 + 2 * causal + padded
    q, k, v, do = (_rand((B, H, N, d), seed + t, sd=0.9) for t in range(4))
    kv_len = np.array([5, 7]) if padded else None
    scale, h = 0.7, 1e-6
    b, hh = 1 if not padded else 0, 1
    q_rows, k_rows = np.array([6, 0, 3]), np.array([2, 6, 4, 0])
    dq, dk, dv = oracle.attention_bwd_sampled_fp64(q, k, v, do, scale, causal, kv_len, "f64",
                                                   b, hh, q_rows, k_rows, chunk=3)
    for name, rows_sel, g in (("q", q_rows, dq), ("k", k_rows, dk), ("v", k_rows, dv)):
        for n, i in enumerate(rows_sel):
            for c in range(d):
                args = {"q": q, "k": k, "v": v}
                base = args[name]
                xp = base.copy(); xp[b, hh, i, c] += h
                xm = base.copy(); xm[b, hh, i, c] -= h
                args[name] = xp
                lp = _loss(args["q"], args["k"], args["v"], do, scale, causal, kv_len)
                args[name] = xm
                lm = _loss(args["q"], args["k"], args["v"], do, scale, causal, kv_len)
                assert abs(g[n, c] - (lp - lm) / (2 * h)) <= 2e-8, (name, i, c)


def test_sampled_backward_equals_dense():
    B, H, N, d = 2, 2, 300, 16
    q, k, v, do = (_rand((B, H, N, d), 9600 + t) for t in range(4))
    kv_len = np.array([300, 123])
    for causal in (False, True):
        dense = oracle.attention_bwd_fp64(q, k, v, do, 0.25, causal, kv_len, kind="f64")
        for b in range(B):
            rows = np.array([0, 1, 64, 122, 123, 299])
            got = oracle.attention_bwd_sampled_fp64(q, k, v, do, 0.25, causal, kv_len, "f64",
                                                    b, 1, rows, rows, chunk=64)
            for g, full in zip(got, dense):
                np.testing.assert_allclose(g, full[b, 1, rows], rtol=0, atol=1e-12)


def test_sampled_backward_query_rows_only():
    B, H, N, d = 1, 1, 200, 8
    q, k, v, do = (_rand((B, H, N, d), 9700 + t) for t in range(4))
    rows = np.array([199, 3, 77, 0, 3])
    for causal in (False, True):
        dense = oracle.attention_bwd_fp64(q, k, v, do, 0.3, causal, None, kind="f64")
        dq, dk, dv = oracle.attention_bwd_sampled_fp64(q, k, v, do, 0.3, causal, None, "f64",
                                                       0, 0, rows, [], chunk=2)
        np.testing.assert_allclose(dq, dense[0][0, 0, rows], rtol=0, atol=1e-12)
        assert dk.shape == (0, d) and dv.shape == (0, d)


def test_sampled_backward_late_keys_causal():
    # under the causal mask only rows i >= j reach key j: selecting late keys
    # visits only late rows, with the same result as the dense backward
    B, H, N, d = 1, 1, 260, 8
    q, k, v, do = (_rand((B, H, N, d), 9800 + t) for t in range(4))
    dense = oracle.attention_bwd_fp64(q, k, v, do, 0.4, True, None, kind="f64")
    keys = np.array([259, 200, 230])
    rows = np.array([5, 250])
    got = oracle.attention_bwd_sampled_fp64(q, k, v, do, 0.4, True, None, "f64", 0, 0, rows, keys,
                                            chunk=16)
    np.testing.assert_allclose(got[0], dense[0][0, 0, rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[1], dense[1][0, 0, keys], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[2], dense[2][0, 0, keys], rtol=0, atol=1e-12)


def test_e4m3_decoder_known_patterns():
    bits = np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x39, 0x7E, 0xB8, 0x80, 0x30, 0x44, 0xFE], dtype=np.uint8)
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.125, 448.0, -1.0, -0.0, 0.5, 3.0, -448.0]
    got = oracle.decode_e4m3_bits(bits)
    np.testing.assert_array_equal(got, want)
    assert np.isnan(oracle.decode_e4m3_bits(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_e4m3_decoder_matches_torch_on_all_patterns():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    bits = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(bits.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3_bits(bits)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def test_fp8_attention_is_attention_of_the_decoded_inputs():
    """Brute force on the exactly decoded, rescaled inputs; the magnitude output
    is the attention of |V|, which bounds |O| elementwise."""
    rng = np.random.default_rng(77)
    B, H, N, d = 1, 2, 9, 4
    # every sign, subnormals included, magnitudes below 4 (exponent field <= 8)
    finite = np.array([b for b in range(256) if ((b >> 3) & 0xF) <= 8], dtype=np.uint8)
    q8, k8, v8 = (rng.choice(finite, size=(B, H, N, d)) for _ in range(3))
    ds = (0.25, 0.5, 2.0)
    out, mag = oracle.attention_fp8_fp64(q8, k8, v8, ds, 0.1, True, None, magnitude=True)
    dec = oracle.decode_e4m3_bits
    Q, K, V = dec(q8) * 0.25, dec(k8) * 0.5, dec(v8) * 2.0
    want = brute_force(Q, K, V, 0.1, True, None)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)
    assert (np.abs(out) <= mag + 1e-12).all()
