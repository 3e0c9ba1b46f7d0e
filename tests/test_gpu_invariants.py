"""GPU edge cases and invariants of the attention path, through the C ABI.

Closed forms and invariants of the definition (constant values, zero scale,
masked keys contributing nothing, fully masked rows), run-to-run determinism,
stream ordering, a negative scale, an input that forces the running maximum to
grow on every key tile, inputs whose probabilities overflow the first tile's
exponent shift (exp2 itself, or only their products with V), and the largest
supported tensor size.
"""

import math
import sys

import numpy as np
import pytest
import torch

from exact_long_sequence_amd import attnio
from exact_long_sequence_amd.inputs import make_inputs, sample_rows

from .parity_util import compare, gpu_rows, oracle_rows, run_gpu

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _fn(dtype):
    return attnio.attn_fwd if dtype == "bf16" else attnio.attn_fwd_f32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_poisoned_padding_keys_do_not_leak(dtype, causal):
    """Keys at or past kv_len hold NaN: O must be finite and bit-identical to the
    run with ordinary values there (those rows are never loaded)."""
    B, H, N, d = 3, 2, 700, 128
    _log(f"poison dtype={dtype} causal={causal}")
    q, k, v, _ = make_inputs(B, H, N, d, dtype, seed=31)
    kv = torch.tensor([N, 333, 129], dtype=torch.int32)
    qd, kd, vd, kvd = q.to(DEV), k.to(DEV), v.to(DEV), kv.to(DEV)
    base = _fn(dtype)(qd, kd, vd, causal=causal, kv_len=kvd)
    kp, vp = kd.clone(), vd.clone()
    for b in range(B):
        kp[b, :, int(kv[b]):] = float("nan")
        vp[b, :, int(kv[b]):] = float("nan")
    pois = _fn(dtype)(qd, kp, vp, causal=causal, kv_len=kvd)
    torch.cuda.synchronize()
    assert torch.isfinite(pois.float()).all()
    assert torch.equal(base.view(torch.int16) if dtype == "bf16" else base.view(torch.int32),
                       pois.view(torch.int16) if dtype == "bf16" else pois.view(torch.int32))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bitwise_determinism(d, causal):
    """Run-to-run bitwise equality over 24 calls, alternating between two
    output buffers (a stale buffer cannot pass for a fresh one) with the
    default-launch-order work of a different call in between."""
    q, k, v, kv = make_inputs(2, 8, 3000, d, "bf16", seed=32, padded=True)
    qd, kd, vd, kvd = q.to(DEV), k.to(DEV), v.to(DEV), kv.to(DEV)
    ref = attnio.attn_fwd(qd, kd, vd, causal=causal, kv_len=kvd)
    outs = [torch.full_like(qd, float("nan")) for _ in range(2)]
    other = torch.empty_like(qd)
    for i in range(24):
        o = outs[i % 2]
        o.fill_(float("nan"))
        attnio.attn_fwd(qd, kd, vd, causal=causal, kv_len=kvd, out=o)
        attnio.attn_fwd(kd, qd, vd, causal=not causal, out=other)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), f"call {i}"


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_reproduce_the_constant(causal):
    """V rows all equal c: every row with a visible key returns c (bf16 P, and l
    summed over the same rounded P, so only fp32 accumulation error remains)."""
    B, H, N, d = 1, 3, 1500, 128
    q, k, _, _ = make_inputs(B, H, N, d, "bf16", seed=33, q_mul=4.0)
    c = (torch.randn(d, generator=torch.Generator().manual_seed(5))).to(torch.bfloat16)
    v = c.expand(B, H, N, d).contiguous()
    o = attnio.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    err = (o.float().cpu() - c.float()).abs().max().item()
    assert err <= 1e-2, err   # bf16 output rounding of c itself is exact; fp32 sums add ~1e-6


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_scale_is_prefix_mean(dtype):
    B, H, N, d = 1, 2, 900, 64
    q, k, v, _ = make_inputs(B, H, N, d, dtype, seed=34)
    o = _fn(dtype)(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=0.0)
    torch.cuda.synchronize()
    v64 = v.double()
    want = torch.cumsum(v64, dim=2) / torch.arange(1, N + 1, dtype=torch.float64)[None, None, :, None]
    err = (o.double().cpu() - want).abs().max().item()
    assert err <= (2e-2 if dtype == "bf16" else 1e-5), err


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fully_masked_rows_are_zero_and_kv_len_clamps(dtype):
    B, H, N, d = 3, 2, 200, 128
    q, k, v, _ = make_inputs(B, H, N, d, dtype, seed=35)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o = _fn(dtype)(qd, kd, vd, kv_len=torch.tensor([0, -5, 10 ** 6], dtype=torch.int32))
    full = _fn(dtype)(qd, kd, vd)
    none = _fn(dtype)(qd, kd, vd, kv_len=torch.tensor([N, N, N], dtype=torch.int32))
    torch.cuda.synchronize()
    assert (o[0] == 0).all() and (o[1] == 0).all()
    assert torch.equal(o[2], full[2])
    assert torch.equal(full, none)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_negative_scale(dtype):
    B, H, N, d = 1, 2, 513, 128
    q, k, v, kv = make_inputs(B, H, N, d, dtype, seed=36, padded=True)
    scale = -0.3
    out = run_gpu(q, k, v, True, kv, scale, dtype)
    want = oracle_rows(q, k, v, True, kv, scale, dtype)
    compare(gpu_rows(out), want, dtype, "negative scale")


def test_running_max_grows_every_tile():
    """Q_i = u, K_j = t_j u with t_j increasing: each key tile raises every
    row's maximum by far more than the lazy-rescale threshold."""
    N, d = 1200, 128
    g = torch.Generator().manual_seed(37)
    u = torch.randn(d, generator=g)
    u = u / u.norm() * 4.0
    t = torch.linspace(-2.0, 6.0, N)
    q = u.expand(1, 1, N, d).to(torch.bfloat16).contiguous()
    k = (t[:, None] * u[None, :])[None, None].to(torch.bfloat16).contiguous()
    v = torch.randn(1, 1, N, d, generator=g).to(torch.bfloat16)
    for causal in (False, True):
        out = run_gpu(q, k, v, causal, None, 1.0, "bf16")
        want = oracle_rows(q, k, v, causal, None, 1.0, "bf16")
        compare(gpu_rows(out), want, "bf16", f"ramp causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_probability_overflow_recomputed(d, causal):
    """Keys 300.. score about 128 (x log2 e = 185 in the exponent) above the
    first key tile on every even row, so the exponent shift taken from that
    tile overflows exp2 there; odd rows stay small.  With the row sum formed
    after the P x V (d = 128) the overflow is seen one tile late and the
    workgroup recomputes its rows with the shift checked before every tile;
    with the row sum formed before it (d = 64) the tile is recomputed at once.
    Either way O must match the oracle on every row, overflowing or not."""
    N = 1000
    _log(f"overflow d={d} causal={causal}")
    g = torch.Generator().manual_seed(39)
    qs, ks = [], []
    for h in range(2):
        u = torch.randn(d, generator=g)
        u = u / u.norm() * 4.0
        t = 0.1 * torch.randn(N, generator=g)
        t[300:] += 8.0
        s = torch.where(torch.arange(N) % 2 == 0, 1.0, 0.05)
        qs.append(s[:, None] * u[None, :])
        ks.append(t[:, None] * u[None, :])
    q = torch.stack(qs)[None].to(torch.bfloat16).contiguous()
    k = torch.stack(ks)[None].to(torch.bfloat16).contiguous()
    v = torch.randn(1, 2, N, d, generator=g).to(torch.bfloat16)
    out = run_gpu(q, k, v, causal, None, 1.0, "bf16")
    want = oracle_rows(q, k, v, causal, None, 1.0, "bf16")
    compare(gpu_rows(out), want, "bf16", f"overflow d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_finite_probability_overflow_recomputed(d, causal):
    """One or two keys per head score 88 (x log2 e = 126.96 in the exponent)
    above every other key on even rows, whose scores are all exactly 0.  The
    exponent shift taken from the first key tile is then 0, the spike's
    probability 2^126.96 is finite in bf16 and fp32, and so is the tile's row
    sum, but its product with |V| = 4 overflows fp32.  The fast pass must send
    the workgroup to the safe pass (d = 128: the row sum is tested after the
    tile's P x V) or recompute the tile before its P x V (d = 64); O must be
    finite and match the oracle on every row."""
    N = 1000
    _log(f"finite-P overflow d={d} causal={causal}")
    g = torch.Generator().manual_seed(41)
    q = torch.zeros(1, 2, N, d)
    q[..., 0] = torch.where(torch.arange(N) % 2 == 0, 1.0, 0.05)
    k = torch.zeros(1, 2, N, d)
    spikes = {0: (130, 700), 1: (500,)}
    v = torch.randn(1, 2, N, d, generator=g)
    for h, js in spikes.items():
        for j in js:
            k[0, h, j, 0] = 88.0
            v[0, h, j] = 4.0 * torch.sign(torch.randn(d, generator=g))
    q, k, v = (t.to(torch.bfloat16).contiguous() for t in (q, k, v))
    out = run_gpu(q, k, v, causal, None, 1.0, "bf16")
    want = oracle_rows(q, k, v, causal, None, 1.0, "bf16")
    compare(gpu_rows(out), want, "bf16", f"finite-P overflow d={d} causal={causal}")


def test_non_default_stream_ordering():
    q, k, v, _ = make_inputs(1, 4, 2048, 128, "bf16", seed=38)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ref = attnio.attn_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = torch.empty_like(qd)
        for _ in range(3):
            attnio.attn_fwd(qd, kd, vd, causal=True, out=out)
    s.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_binding_rejects_bad_arguments():
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(TypeError):
        attnio.attn_fwd(x.float(), x.float(), x.float())
    with pytest.raises(ValueError):
        attnio.attn_fwd(x, x, x.transpose(2, 3))
    y = torch.zeros(1, 1, 8, 96, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError, match="head size"):
        attnio.attn_fwd(y, y, y)
    with pytest.raises(RuntimeError, match="overlaps"):
        attnio.attn_fwd(x, x, x, out=x)


def test_largest_supported_size():
    """B*H*N*d = 2^31 - 2^18 elements per tensor (4 GiB of bf16 each): the
    int32 element bound of the interface, checked on sampled rows."""
    B, H, N, d = 1, 8191, 2048, 128
    assert B * H * N * d < 2 ** 31
    _log("largest size: generating inputs on the GPU")
    g = torch.Generator(device=DEV).manual_seed(39)
    q = torch.randn(B, H, N, d, generator=g, device=DEV, dtype=torch.bfloat16)
    k = torch.randn(B, H, N, d, generator=g, device=DEV, dtype=torch.bfloat16)
    v = torch.randn(B, H, N, d, generator=g, device=DEV, dtype=torch.bfloat16)
    scale = float(np.float32(1 / math.sqrt(d)))
    o = attnio.attn_fwd(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    rows = sample_rows(B, H, N, 256, seed=39)
    heads = np.unique(rows // N)
    import oracle
    from exact_long_sequence_amd.inputs import oracle_view
    got_all, want_all = [], []
    for hh in heads:
        sel = rows[rows // N == hh] % N
        qh, kh, vh = (t[0, int(hh)].cpu()[None, None] for t in (q, k, v))
        want = oracle.attention_fp64(oracle_view(qh), oracle_view(kh), oracle_view(vh), scale, True,
                                     None, kind="bf16", rows=sel)
        got = o[0, int(hh)][torch.as_tensor(sel, device=DEV)].float().cpu().numpy().astype(np.float64)
        got_all.append(got)
        want_all.append(want)
    compare(np.concatenate(got_all), np.concatenate(want_all), "bf16", "largest size")
