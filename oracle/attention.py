"""Plain fp64 CPU oracle for exact self-attention (forward, its log-sum-exp
side output, and the backward gradients).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP library and imports neither torch
nor the package; it takes plain numpy arrays.

What it computes is the attention operator graph written out literally, in
three materialising steps (scores, mask + softmax, weighted sum of values):

    Scores = scale * Q x K^T          ("From Attention Graph to FlashAttention -
    Scores = Mask(Scores)              A Memory-Centric Compilation Approach in
    Scores = Softmax(Scores)           AICF", section 1, the basic attention
    Output = Scores x V                operator graph; section 5 repeats it as
                                       the pattern MatMul / Mask / Softmax /
                                       MatMul)

The score matrix is materialised here on purpose, one chunk of query rows at a
time: this is the naive form whose score / softmax / probability intermediates
(same page, section 1) the streamed kernel avoids.  Softmax is shifted by the
row maximum before exponentiation, which leaves the mathematical result
unchanged and only keeps fp64 exp from overflowing.

Readings of points the pages leave open (each also listed in the design notes):
  * layout: contiguous [B, H, N, d], d innermost;
  * causal mask: query i may attend to key j iff j <= i;
  * key padding: kv_len[b] masks keys j >= kv_len[b] only; every query row is
    still produced;
  * a row with no allowed key (only possible when kv_len[b] == 0) is all zeros;
  * scale is the fp32 value the caller passes, widened exactly to fp64;
  * bf16 inputs arrive as their raw 16-bit patterns and are widened exactly.

Every function here is pinned by tests/test_oracle.py against brute force on
tiny inputs, closed forms and invariants (softmax rows sum to one, constant
values give that constant, masked keys contribute nothing, ...).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "decode_bf16_bits",
    "to_fp64",
    "effective_kv_len",
    "allowed_mask",
    "attention_fp64",
    "attention_rows_fp64",
    "attention_full_fp64",
    "attention_lse_fp64",
    "attention_bwd_fp64",
    "attention_bwd_rows_fp64",
    "attention_bwd_sampled_fp64",
    "decode_e4m3_bits",
    "attention_fp8_fp64",
]


def decode_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bit patterns (uint16) to float64, exactly.

    A bfloat16 value is the upper half of the IEEE-754 binary32 pattern, so
    shifting the 16 bits into the top of a 32-bit word reproduces the binary32
    number bit for bit; binary32 -> binary64 is exact.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError(f"bf16 bits must be uint16, got {b.dtype}")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_e4m3_bits(bits: np.ndarray) -> np.ndarray:
    """Widen raw 8-bit float patterns of the OCP E4M3 ("e4m3fn") format to
    float64, exactly: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 holds the subnormals m/8 * 2^-6; the all-ones pattern
    S.1111.111 is NaN and there are no infinities (largest finite 448)."""
    b = np.asarray(bits)
    if b.dtype != np.uint8:
        raise TypeError(f"e4m3 bits must be uint8, got {b.dtype}")
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = ((b >> 3) & 0xF).astype(np.int64)
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    nan = (e == 15) & (m == 7)
    return np.where(nan, np.nan, sign * mag)


def to_fp64(x: np.ndarray, kind: str) -> np.ndarray:
    """Exact widening of an input tensor: kind is 'bf16' (uint16 bits), 'f32' or 'f64'."""
    if kind == "bf16":
        return decode_bf16_bits(x)
    if kind == "f32":
        a = np.asarray(x)
        if a.dtype != np.float32:
            raise TypeError(f"f32 input must be float32, got {a.dtype}")
        return a.astype(np.float64)
    if kind == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown input kind {kind!r}")


def effective_kv_len(kv_len, B: int, N: int) -> np.ndarray:
    """Per-batch number of visible keys: kv_len clamped to [0, N], or N when absent."""
    if kv_len is None:
        return np.full(B, N, dtype=np.int64)
    kl = np.asarray(kv_len, dtype=np.int64).reshape(-1)
    if kl.shape[0] != B:
        raise ValueError(f"kv_len has {kl.shape[0]} entries, expected B={B}")
    return np.clip(kl, 0, N)


def allowed_mask(rows: np.ndarray, n_keys: int, L: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), n_keys]: key j is visible to query row i iff j < L and
    (not causal or j <= i).  This is the optional Mask step of the operator graph."""
    j = np.arange(n_keys)[None, :]
    ok = j < L
    if causal:
        ok = ok & (j <= np.asarray(rows)[:, None])
    return ok


def _softmax_rows(S: np.ndarray, ok: np.ndarray):
    """Row softmax of S restricted to the allowed entries; masked entries are -inf
    before normalisation and exactly 0 after.  Rows with no allowed entry give an
    all-zero probability row and lse = -inf.  Returns (P, lse)."""
    S = np.where(ok, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    E = np.exp(S - m_safe)  # exp(-inf) == 0 exactly on masked entries
    l = E.sum(axis=1, keepdims=True)
    l_safe = np.where(empty, 1.0, l)
    P = E / l_safe
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return P, lse[:, 0]


def attention_rows_fp64(Qf: np.ndarray, Kf: np.ndarray, Vf: np.ndarray, rows,
                        scale: float, causal: bool, L: int, chunk: int = 1024,
                        want_p: bool = False):
    """Attention output for selected query rows of ONE (batch, head) slice.

    Qf, Kf, Vf: float64 [N, d].  rows: int array of query indices.  L: visible
    key count for this batch.  Returns O [len(rows), d] (and P, lse if want_p).
    Steps: scores = s * Q[rows] K^T; mask; softmax; P V -- materialised per chunk.
    """
    rows = np.asarray(rows, dtype=np.int64)
    n_keys = Kf.shape[0]
    s64 = float(np.float32(scale))
    out = np.empty((rows.shape[0], Vf.shape[1]), dtype=np.float64)
    Ps, lses = [], []
    for c0 in range(0, rows.shape[0], chunk):
        r = rows[c0:c0 + chunk]
        S = s64 * (Qf[r] @ Kf.T)                       # Scores = Q x K^T (scaled)
        ok = allowed_mask(r, n_keys, L, causal)         # Mask
        P, lse = _softmax_rows(S, ok)                   # Softmax
        out[c0:c0 + chunk] = P @ Vf                     # Output = Scores x V
        if want_p:
            Ps.append(P)
            lses.append(lse)
    if want_p:
        return out, np.concatenate(Ps, axis=0), np.concatenate(lses)
    return out


def attention_fp64(q, k, v, scale: float, causal: bool = False, kv_len=None,
                   kind: str = "bf16", rows=None, chunk: int = 1024) -> np.ndarray:
    """Exact attention forward in fp64 for [B, H, N, d] inputs.

    q, k, v: arrays of the given kind ('bf16' = uint16 bit patterns, 'f32', 'f64').
    rows: None for every row (returns [B, H, N, d]), or an int array of flat
    (b*H + h)*N + i indices (returns [len(rows), d] in the given order).
    kv_len: None or a length-B integer array (clamped to [0, N]).
    """
    qa, ka, va = np.asarray(q), np.asarray(k), np.asarray(v)
    if qa.ndim != 4 or qa.shape != ka.shape or qa.shape != va.shape:
        raise ValueError(f"q/k/v must share one [B,H,N,d] shape, got {qa.shape} {ka.shape} {va.shape}")
    B, H, N, d = qa.shape
    Ls = effective_kv_len(kv_len, B, N)
    if rows is None:
        out = np.empty((B, H, N, d), dtype=np.float64)
        for b in range(B):
            for h in range(H):
                Qf = to_fp64(qa[b, h], kind)
                Kf = to_fp64(ka[b, h], kind)
                Vf = to_fp64(va[b, h], kind)
                out[b, h] = attention_rows_fp64(Qf, Kf, Vf, np.arange(N), scale, causal,
                                                int(Ls[b]), chunk)
        return out
    flat = np.asarray(rows, dtype=np.int64).reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= B * H * N):
        raise ValueError("row index out of range")
    out = np.empty((flat.shape[0], d), dtype=np.float64)
    bh = flat // N
    for s in np.unique(bh):
        sel = np.nonzero(bh == s)[0]
        b, h = divmod(int(s), H)
        Qf = to_fp64(qa[b, h], kind)
        Kf = to_fp64(ka[b, h], kind)
        Vf = to_fp64(va[b, h], kind)
        out[sel] = attention_rows_fp64(Qf, Kf, Vf, flat[sel] % N, scale, causal,
                                       int(Ls[b]), chunk)
    return out


def attention_full_fp64(q, k, v, scale: float, causal: bool = False, kv_len=None,
                        kind: str = "f64"):
    """Tiny-case variant that also returns the probability matrix and the
    log-sum-exp of each row: (O [B,H,N,d], P [B,H,N,N], lse [B,H,N])."""
    qa, ka, va = np.asarray(q), np.asarray(k), np.asarray(v)
    B, H, N, d = qa.shape
    Ls = effective_kv_len(kv_len, B, N)
    O = np.empty((B, H, N, d))
    P = np.empty((B, H, N, N))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o, p, l = attention_rows_fp64(to_fp64(qa[b, h], kind), to_fp64(ka[b, h], kind),
                                          to_fp64(va[b, h], kind), np.arange(N), scale,
                                          causal, int(Ls[b]), want_p=True)
            O[b, h], P[b, h], lse[b, h] = o, p, l
    return O, P, lse


def attention_lse_fp64(q, k, v, scale: float, causal: bool = False, kv_len=None,
                       kind: str = "bf16", rows=None, chunk: int = 1024) -> np.ndarray:
    """Log-sum-exp of each query row's scaled, masked scores, in fp64:
    lse_i = ln sum_j exp(scale * q_i . k_j) over the keys j visible to row i, or
    -inf for a row with no visible key.  This is the per-row statistic the
    backward pass recomputes the probabilities from ("IO-Aware Algorithms",
    How it works, recomputation).  rows: None for [B, H, N], or flat
    (b*H + h)*N + i indices (returns [len(rows)])."""
    qa, ka, va = np.asarray(q), np.asarray(k), np.asarray(v)
    B, H, N, d = qa.shape
    Ls = effective_kv_len(kv_len, B, N)
    flat = (np.arange(B * H * N, dtype=np.int64) if rows is None
            else np.asarray(rows, dtype=np.int64).reshape(-1))
    if flat.size and (flat.min() < 0 or flat.max() >= B * H * N):
        raise ValueError("row index out of range")
    out = np.empty(flat.shape[0], dtype=np.float64)
    bh = flat // N
    for s in np.unique(bh):
        sel = np.nonzero(bh == s)[0]
        b, h = divmod(int(s), H)
        _, _, lse = attention_rows_fp64(to_fp64(qa[b, h], kind), to_fp64(ka[b, h], kind),
                                        to_fp64(va[b, h], kind), flat[sel] % N, scale, causal,
                                        int(Ls[b]), chunk, want_p=True)
        out[sel] = lse
    return out if rows is not None else out.reshape(B, H, N)


def attention_bwd_rows_fp64(Qf: np.ndarray, Kf: np.ndarray, Vf: np.ndarray, dOf: np.ndarray,
                            scale: float, causal: bool, L: int):
    """Gradients of one (batch, head) slice, all rows, in fp64.

    With S = s Q K^T masked, P = softmax(S) and O = P V, the loss gradient dO
    gives (the chain rule through the operator graph, as the backward pass of
    "IO-Aware Algorithms", How it works, recomputes it from Q, K, V):
        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - rowsum(P * dP))        (softmax Jacobian, row by row)
        dQ = s dS K,   dK = s dS^T Q
    P is materialised here on purpose; masked entries are exactly 0."""
    N = Qf.shape[0]
    s64 = float(np.float32(scale))
    S = s64 * (Qf @ Kf.T)
    ok = allowed_mask(np.arange(N), Kf.shape[0], L, causal)
    P, _ = _softmax_rows(S, ok)
    dV = P.T @ dOf
    dP = dOf @ Vf.T
    Dr = (P * dP).sum(axis=1, keepdims=True)
    dS = P * (dP - Dr)
    dQ = s64 * (dS @ Kf)
    dK = s64 * (dS.T @ Qf)
    return dQ, dK, dV


def attention_bwd_fp64(q, k, v, do, scale: float, causal: bool = False, kv_len=None,
                       kind: str = "bf16"):
    """Exact attention backward in fp64 for [B, H, N, d] inputs: returns
    (dQ, dK, dV), each float64 [B, H, N, d].  q, k, v, do are of the given kind
    ('bf16' uint16 bit patterns, 'f32' or 'f64').  Keys past kv_len get zero
    gradients; rows without a visible key contribute nothing."""
    qa, ka, va, da = (np.asarray(t) for t in (q, k, v, do))
    if qa.ndim != 4 or not (qa.shape == ka.shape == va.shape == da.shape):
        raise ValueError("q, k, v, do must share one [B,H,N,d] shape")
    B, H, N, d = qa.shape
    Ls = effective_kv_len(kv_len, B, N)
    dQ = np.empty((B, H, N, d)); dK = np.empty((B, H, N, d)); dV = np.empty((B, H, N, d))
    for b in range(B):
        for h in range(H):
            dQ[b, h], dK[b, h], dV[b, h] = attention_bwd_rows_fp64(
                to_fp64(qa[b, h], kind), to_fp64(ka[b, h], kind), to_fp64(va[b, h], kind),
                to_fp64(da[b, h], kind), scale, causal, int(Ls[b]))
    return dQ, dK, dV


def attention_bwd_sampled_fp64(q, k, v, do, scale: float, causal: bool, kv_len, kind: str,
                               b: int, h: int, q_rows, k_rows, chunk: int = 512):
    """Selected gradient rows of ONE (batch, head) slice, for sizes where the
    dense form does not fit: returns (dQ[q_rows], dK[k_rows], dV[k_rows]).

    The same definitions as attention_bwd_rows_fp64, taken over chunks of query
    rows so that only a chunk x N block of P, dP and dS ever exists.  A row's
    softmax, D_i = rowsum(P * dP) and dS need only that row, so each chunk
    completes its rows; the key-side gradients are sums over query rows,
        dV_j = sum_i P_ij dO_i,    dK_j = s sum_i dS_ij Q_i,
    accumulated chunk by chunk for the selected keys j only.  Rows that
    contribute nothing to what was asked for (rows before the first selected
    key under the causal mask, unselected rows when no key is selected) are
    never visited."""
    qa, ka, va, da = (np.asarray(t) for t in (q, k, v, do))
    B, H, N, d = qa.shape
    L = int(effective_kv_len(kv_len, B, N)[b])
    Qf, Kf, Vf, dOf = (to_fp64(t[b, h], kind) for t in (qa, ka, va, da))
    s64 = float(np.float32(scale))
    q_rows = np.asarray(q_rows, dtype=np.int64).reshape(-1)
    k_rows = np.asarray(k_rows, dtype=np.int64).reshape(-1)
    dQ = np.zeros((q_rows.size, d))
    dK = np.zeros((k_rows.size, d))
    dV = np.zeros((k_rows.size, d))
    n_keys = min(L, N)
    # a query row's own gradient needs only that row; key j's gradients need
    # every row that sees key j: all rows, or under the causal mask rows i >= j
    visit = np.unique(q_rows)
    if k_rows.size:
        first = int(k_rows.min()) if causal else 0
        visit = np.union1d(visit, np.arange(first, N))
    for c0 in range(0, visit.size, chunk):
        r = visit[c0:c0 + chunk]
        # keys a row of this chunk can see: j < L, and j <= i when causal
        kmax = min(n_keys, int(r.max()) + 1) if causal else n_keys
        if kmax == 0:
            continue
        S = s64 * (Qf[r] @ Kf[:kmax].T)
        ok = allowed_mask(r, kmax, L, causal)
        P, _ = _softmax_rows(S, ok)
        dP = dOf[r] @ Vf[:kmax].T
        Dr = (P * dP).sum(axis=1, keepdims=True)
        dS = P * (dP - Dr)
        pos = {int(i): n for n, i in enumerate(r)}
        for n, i in enumerate(q_rows):
            if int(i) in pos:
                dQ[n] = s64 * (dS[pos[int(i)]] @ Kf[:kmax])
        ksel = np.nonzero(k_rows < kmax)[0]
        if ksel.size:
            cols = k_rows[ksel]
            dV[ksel] += P[:, cols].T @ dOf[r]
            dK[ksel] += s64 * (dS[:, cols].T @ Qf[r])
    return dQ, dK, dV


def attention_fp8_fp64(q8, k8, v8, descale, scale: float, causal: bool = False, kv_len=None,
                       rows=None, magnitude: bool = False):
    """Exact attention of fp8 (OCP E4M3) inputs in fp64.

    q8, k8, v8: uint8 bit patterns [B, H, N, d]; descale = (q_s, k_s, v_s): the
    fp32 factors that turn each tensor's fp8 values into the real inputs
    (x = fp8(bits) * s).  The real inputs are formed exactly in fp64 and the
    attention operator graph is applied to them as in attention_fp64.

    magnitude: also return M = |P| |V| (the probabilities applied to the
    absolute values), same shape as the output: the scale of the error that
    rounding the probabilities to fp8 can cause in each output element."""
    qs, ks, vs = (float(np.float32(x)) for x in descale)
    Q = decode_e4m3_bits(np.asarray(q8)) * qs
    K = decode_e4m3_bits(np.asarray(k8)) * ks
    V = decode_e4m3_bits(np.asarray(v8)) * vs
    out = attention_fp64(Q, K, V, scale, causal, kv_len, kind="f64", rows=rows)
    if not magnitude:
        return out
    mag = attention_fp64(Q, K, np.abs(V), scale, causal, kv_len, kind="f64", rows=rows)
    return out, mag
