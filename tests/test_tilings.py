"""Every compiled tiling of the bf16 forward, run explicitly through
attn_fwd_tiled (C ABI), against the fp64 oracle.

The forward runs the tiling the I/O model picks; the other compiled tilings
exist to check that choice by measurement, so each must compute the same
function.  Every row of a small sweep (ragged N, causal, key padding from 0)
is compared with the oracle at the bf16 tolerance; keys past kv_len are
NaN-poisoned and must not leak; a negative scale (each kernel's other
instantiation) is checked the same way; an input whose probability overflows the
first tile's shift without overflowing exp2 (one key 126.96 above it in the
base-2 domain, |V| = 4) must be recomputed; the picked tiling must be
bitwise what attn_fwd returns.
"""

import sys

import numpy as np
import pytest
import torch

from exact_long_sequence_amd import attnio
from exact_long_sequence_amd.inputs import make_inputs

from .parity_util import compare, gpu_rows, oracle_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _tilings():
    return [(i, attnio.attn_tiling_get(i)) for i in range(attnio.attn_tiling_count())]


def _ids():
    out = []
    for i, t in _tilings():
        out.append(f"{i}-d{t['d']}-BM{t['BM']}-BN{t['BN']}-qb{t['qb']}-wpc{t['wg_per_cu']}"
                   f"-{'pp' if t['pingpong'] else 'seq'}-{'rsv' if not t['rowsum_mfma'] else ('rss' if t['rowsum_in_stream'] else 'rsw')}"
                   f"{'-m16' if t['mfma16'] else ''}")
    return out


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("index", range(attnio.attn_tiling_count()), ids=_ids())
def test_tiling_matches_oracle(index):
    t = attnio.attn_tiling_get(index)
    d = t["d"]
    for N in (1, 65, 300, 1000, 1100):
        for causal in (False, True):
            for padded in (False, True):
                _log(f"tiling {index} d={d} N={N} causal={causal} padded={padded}")
                q, k, v, kv = make_inputs(2, 3, N, d, "bf16", seed=61 + N, padded=padded, kv_lo=0)
                qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
                kvd = None if kv is None else kv.to(DEV)
                if kv is not None:   # poison what no query may see
                    for b in range(2):
                        kd[b, :, int(kv[b]):] = float("nan")
                        vd[b, :, int(kv[b]):] = float("nan")
                out = attnio.attn_fwd_tiled(qd, kd, vd, index, causal=causal, kv_len=kvd)
                torch.cuda.synchronize()
                want = oracle_rows(q, k, v, causal, kv, float(np.float32(1 / np.sqrt(d))), "bf16")
                compare(gpu_rows(out), want, "bf16", f"tiling {index} N={N} causal={causal} padded={padded}")


@pytest.mark.parametrize("index", range(attnio.attn_tiling_count()), ids=_ids())
def test_tiling_negative_scale(index):
    """A negative scale takes each kernel's other instantiation (row minimum of
    the raw scores, masked scores +inf): every row, causal x key padding."""
    t = attnio.attn_tiling_get(index)
    d = t["d"]
    scale = -float(np.float32(0.7 / np.sqrt(d)))
    for N in (300, 1100):
        for causal in (False, True):
            for padded in (False, True):
                _log(f"tiling {index} d={d} N={N} causal={causal} padded={padded} scale={scale}")
                q, k, v, kv = make_inputs(2, 3, N, d, "bf16", seed=71 + N, padded=padded, kv_lo=0)
                kvd = None if kv is None else kv.to(DEV)
                out = attnio.attn_fwd_tiled(q.to(DEV), k.to(DEV), v.to(DEV), index, causal=causal, kv_len=kvd,
                                            scale=scale)
                torch.cuda.synchronize()
                want = oracle_rows(q, k, v, causal, kv, scale, "bf16")
                compare(gpu_rows(out), want, "bf16", f"tiling {index} N={N} causal={causal} padded={padded} neg")


@pytest.mark.parametrize("index", range(attnio.attn_tiling_count()), ids=_ids())
def test_tiling_finite_probability_overflow(index):
    t = attnio.attn_tiling_get(index)
    d, N = t["d"], 1100
    _log(f"tiling {index} finite-P overflow")
    g = torch.Generator().manual_seed(71)
    q = torch.zeros(1, 2, N, d)
    q[..., 0] = torch.where(torch.arange(N) % 2 == 0, 1.0, 0.05)
    k = torch.zeros(1, 2, N, d)
    v = torch.randn(1, 2, N, d, generator=g)
    for h, js in {0: (130, 700), 1: (600,)}.items():
        for j in js:
            k[0, h, j, 0] = 88.0
            v[0, h, j] = 4.0 * torch.sign(torch.randn(d, generator=g))
    q, k, v = (x.to(torch.bfloat16).contiguous() for x in (q, k, v))
    for causal in (False, True):
        out = attnio.attn_fwd_tiled(q.to(DEV), k.to(DEV), v.to(DEV), index, causal=causal, scale=1.0)
        torch.cuda.synchronize()
        want = oracle_rows(q, k, v, causal, None, 1.0, "bf16")
        compare(gpu_rows(out), want, "bf16", f"tiling {index} overflow causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_picked_tiling_is_what_attn_fwd_runs(d):
    ev = attnio.attn_tiling_enumerate(d)
    pick = next(e["compiled"] for e in ev if e["compiled"] >= 0)
    q, k, v, kv = make_inputs(1, 4, 2000, d, "bf16", seed=81, padded=True)
    qd, kd, vd, kvd = q.to(DEV), k.to(DEV), v.to(DEV), kv.to(DEV)
    a = attnio.attn_fwd(qd, kd, vd, causal=True, kv_len=kvd)
    b = attnio.attn_fwd_tiled(qd, kd, vd, pick, causal=True, kv_len=kvd)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    bm = attnio.attn_query_tiling(d, True)
    assert bm["BM"] == attnio.attn_tiling_get(pick)["BM"] and bm["BN"] == attnio.attn_tiling_get(pick)["BN"]
