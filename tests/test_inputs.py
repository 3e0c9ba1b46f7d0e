"""CPU checks of the seeded input generators (they hold no attention arithmetic,
but every parity test depends on them being what their docstrings say)."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_long_sequence_amd.inputs import (ROW_WORKLOADS, WORKLOADS, make_fp8_inputs, make_inputs,
                                            quantize_e4m3, row_workload_inputs)


def test_make_inputs_is_seeded_and_rounded():
    a = make_inputs(2, 3, 17, 64, "bf16", seed=5, padded=True)
    b = make_inputs(2, 3, 17, 64, "bf16", seed=5, padded=True)
    for x, y in zip(a[:3], b[:3]):
        assert x.dtype == torch.bfloat16 and torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.equal(a[3], b[3]) and a[3].dtype == torch.int32
    assert ((a[3] >= 17 // 4) & (a[3] <= 17)).all()
    # Q x 8 commutes with the bf16 rounding (a power of two)
    q1 = make_inputs(1, 1, 9, 64, "bf16", seed=3)[0]
    q8 = make_inputs(1, 1, 9, 64, "bf16", seed=3, q_mul=8.0)[0]
    assert torch.equal(q1.float() * 8, q8.float())


def test_quantize_e4m3_round_to_nearest_with_power_of_two_descale():
    g = torch.Generator().manual_seed(11)
    x = torch.randn(4096, generator=g) * 3.7
    bits, s = quantize_e4m3(x)
    assert bits.dtype == torch.uint8
    assert s > 0 and math.log2(s) == int(math.log2(s))        # a power of two
    dec = oracle.decode_e4m3_bits(bits.numpy())
    assert np.isfinite(dec).all() and np.abs(dec).max() <= 448
    y = (x / s).double().numpy()
    assert np.abs(y).max() <= 448
    # nearest representable value: no E4M3 value lies strictly closer to y
    grid = oracle.decode_e4m3_bits(np.arange(256, dtype=np.uint8))
    grid = np.unique(grid[np.isfinite(grid)])
    best = grid[np.abs(grid[None, :] - y[:, None]).argmin(axis=1)]
    np.testing.assert_array_equal(np.abs(dec - y), np.abs(best - y))


def test_make_fp8_inputs_follows_the_fp32_draws():
    q8, k8, v8, ds, kv = make_fp8_inputs(1, 2, 33, 64, seed=21, padded=True)
    q, k, v, kv2 = make_inputs(1, 2, 33, 64, "f32", seed=21, padded=True)
    assert torch.equal(kv, kv2)
    for t8, t, s in zip((q8, k8, v8), (q, k, v), ds):
        dec = oracle.decode_e4m3_bits(t8.numpy()) * s
        # within half a step of E4M3 (2^-4 relative, or the subnormal step)
        err = np.abs(dec - t.double().numpy())
        assert (err <= np.maximum(np.abs(t.double().numpy()) * 2.0 ** -4, 2.0 ** -10 * s) + 1e-12).all()


@pytest.mark.parametrize("name", list(ROW_WORKLOADS))
def test_row_workloads_shapes(name):
    w = ROW_WORKLOADS[name]
    small = type(w)(w.name, w.op, 4, 64, w.param, w.seed)
    x, g, b = row_workload_inputs(small)
    assert x.shape == (4, 64) and x.dtype == torch.bfloat16
    if w.op == "layernorm":
        assert g.shape == (64,) and b.shape == (64,)
    else:
        assert g is None and b is None


def test_workload_table_matches_the_stated_shapes():
    shapes = {n: (w.B, w.H, w.N, w.d, w.dtype, w.causal, w.padded) for n, w in WORKLOADS.items()}
    assert shapes["bf16_causal_h32_n32k_d128"] == (1, 32, 32768, 128, "bf16", True, False)
    assert shapes["single_head_fp32_n1k_d64"] == (1, 1, 1024, 64, "f32", False, False)
    assert shapes["bf16_causal_h8_n128k_d64"] == (1, 8, 131072, 64, "bf16", True, False)
    assert shapes["bf16_padded_b4_h32_n16k_d128_q8"] == (4, 32, 16384, 128, "bf16", False, True)
    assert shapes["bf16_h16_n8k_d128"] == (1, 16, 8192, 128, "bf16", False, False)
