"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and picks rows to check; it holds none of the
attention arithmetic.  Both the HIP path and the fp64 oracle are fed from it:
the oracle receives the rounded bf16 bit patterns (or fp32 arrays) it produces,
so parity never depends on how the numbers were drawn.

Recipe (the pages publish no dataset or test vector; every workload is
synthetic): a CPU torch.Generator seeded with the workload's seed draws Q, K and
V in that order as float32 N(0, 1) tensors of shape [B, H, N, d]; Q is then
multiplied by q_mul (a power of two, so it commutes with rounding) and every
tensor is rounded to bfloat16 (round-to-nearest-even) unless the workload is
fp32.  Key-padding lengths, when the workload has them, are drawn next from the
same generator, uniformly from the inclusive range [N/4, N].
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "quantize_e4m3", "make_fp8_inputs", "make_inputs", "oracle_view", "sample_rows", "RowWorkload",
           "ROW_WORKLOADS", "row_workload_inputs"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "bf16" or "f32"
    causal: bool
    padded: bool        # per-batch key-padding lengths drawn from [N/4, N]
    q_mul: float        # Q multiplier before rounding (peaked softmax when > 1)
    seed: int
    full_check: bool    # oracle checks every row (else a seeded sample)

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to fp32: the value the kernel receives."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "H": self.H, "N": self.N, "d": self.d,
                "dtype": self.dtype, "causal": self.causal, "key_padding": self.padded,
                "q_mul": self.q_mul, "seed": self.seed}


# The five workloads of the exact long-sequence attention study, by shape.
WORKLOADS = {
    "single_head_fp32_n1k_d64": Workload("single_head_fp32_n1k_d64", 1, 1, 1024, 64, "f32",
                                         False, False, 1.0, 1001, True),
    "bf16_h16_n8k_d128": Workload("bf16_h16_n8k_d128", 1, 16, 8192, 128, "bf16",
                                  False, False, 1.0, 1002, True),
    "bf16_causal_h32_n32k_d128": Workload("bf16_causal_h32_n32k_d128", 1, 32, 32768, 128,
                                          "bf16", True, False, 1.0, 1003, False),
    "bf16_causal_h8_n128k_d64": Workload("bf16_causal_h8_n128k_d64", 1, 8, 131072, 64,
                                         "bf16", True, False, 1.0, 1004, False),
    "bf16_padded_b4_h32_n16k_d128_q8": Workload("bf16_padded_b4_h32_n16k_d128_q8", 4, 32, 16384,
                                                128, "bf16", False, True, 8.0, 1005, False),
}


def make_inputs(B: int, H: int, N: int, d: int, dtype: str = "bf16", seed: int = 0,
                padded: bool = False, q_mul: float = 1.0, kv_lo: int | None = None):
    """Draw (q, k, v, kv_len) on the CPU.  kv_len is an int32 tensor [B] or None.

    kv_lo overrides the lower end of the padding range (default N // 4)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if q_mul != 1.0:
        q.mul_(q_mul)
    kv_len = None
    if padded:
        lo = N // 4 if kv_lo is None else kv_lo
        kv_len = torch.randint(lo, N + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    if dtype == "bf16":
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    return q, k, v, kv_len


def workload_inputs(w: Workload):
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.padded, w.q_mul)


def oracle_view(t: torch.Tensor) -> np.ndarray:
    """numpy view for the oracle: uint16 bit patterns for bf16, float32 for fp32."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


# Query-tile heights of the kernels' tilings (rows per workgroup and, for the
# smaller ones, per wave group): rows on both sides of every multiple of these
# up to 1024 are forced into each sample.
TILE_EDGES = (32, 64, 128, 256, 512)


def sample_rows(B: int, H: int, N: int, n_sample: int, seed: int, boundary_bms=TILE_EDGES,
                kv_len=None) -> np.ndarray:
    """Seeded sample of flat (b*H + h)*N + i query-row indices, plus boundary rows.

    Boundary rows, in the first and last (b, h) slices: i in {0, 1, N-2, N-1}
    and i in {k*BM - 1, k*BM} for every BM in boundary_bms and k*BM <= 1024
    (the edges of the query tiles), plus the last tile edges below N.  With key
    padding, also the rows i = L-1 and L of the first head of the batches with
    the smallest and largest length L."""
    total = B * H * N
    rng = np.random.default_rng(int(seed) + 1)
    n = min(n_sample, total)
    picked = rng.choice(total, n, replace=False)
    if isinstance(boundary_bms, int):
        boundary_bms = (boundary_bms,)
    edge_rows = {0, 1, N - 2, N - 1}
    for bm in boundary_bms:
        for e in range(bm, min(N, 1024) + 1, bm):
            edge_rows.update((e - 1, e))
        last = (N - 1) // bm * bm
        edge_rows.update((last - 1, last))
    extra = []
    for (b, h) in {(0, 0), (B - 1, H - 1)}:
        for i in sorted(edge_rows):
            if 0 <= i < N:
                extra.append((b * H + h) * N + i)
    if kv_len is not None:
        kl = np.asarray(kv_len).reshape(-1)
        for b in {int(np.argmin(kl)), int(np.argmax(kl))}:
            for i in (int(kl[b]) - 1, int(kl[b])):
                if 0 <= i < N:
                    extra.append((b * H) * N + i)
    rows = np.unique(np.concatenate([picked, np.asarray(extra, dtype=np.int64)]))
    return rows.astype(np.int64)


@dataclasses.dataclass(frozen=True)
class RowWorkload:
    """A streaming row operator over a bf16 [R, N] matrix."""
    name: str
    op: str          # "softmax" or "layernorm"
    R: int
    N: int
    param: float     # softmax scale or LayerNorm eps
    seed: int

    def describe(self) -> dict:
        return {"workload": self.name, "op": self.op, "R": self.R, "N": self.N,
                "param": self.param, "seed": self.seed, "dtype": "bf16"}


# Row workloads at the attention path's scale: the full score matrix of one
# 32768-row head, and the 131072-token activations of a d=64 x 128-head model
# (hidden size 8192).  Recipe: a seeded CPU torch.Generator draws x as fp32
# N(0, 1) [R, N]; for LayerNorm it then draws gamma = 1 + 0.1 N(0, 1) and
# beta = 0.1 N(0, 1) of length N; everything is rounded to bf16.
ROW_WORKLOADS = {
    "softmax_r32k_n32k": RowWorkload("softmax_r32k_n32k", "softmax", 32768, 32768, 1.0, 1101),
    "layernorm_r128k_n8k": RowWorkload("layernorm_r128k_n8k", "layernorm", 131072, 8192, 1e-5, 1102),
}


def row_workload_inputs(w: RowWorkload):
    """(x, gamma, beta) on the CPU; gamma and beta are None for softmax."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(w.seed))
    x = torch.randn((w.R, w.N), generator=g, dtype=torch.float32).to(torch.bfloat16)
    if w.op == "softmax":
        return x, None, None
    gamma = (1.0 + 0.1 * torch.randn((w.N,), generator=g, dtype=torch.float32)).to(torch.bfloat16)
    beta = (0.1 * torch.randn((w.N,), generator=g, dtype=torch.float32)).to(torch.bfloat16)
    return x, gamma, beta


def quantize_e4m3(x: torch.Tensor):
    """Round an fp32 tensor to OCP E4M3 with one power-of-two descale chosen so
    that the largest magnitude lands at or below 448: returns (uint8 bits,
    descale) with x ~= fp8(bits) * descale.  A power of two keeps the descale
    exact in every precision."""
    amax = float(x.abs().max()) if x.numel() else 0.0
    s = 2.0 ** math.ceil(math.log2(amax / 448.0)) if amax > 0 else 1.0
    q = (x / s).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), s


def make_fp8_inputs(B: int, H: int, N: int, d: int, seed: int = 0, padded: bool = False,
                    q_mul: float = 1.0, kv_lo: int | None = None):
    """fp8 inputs: the fp32 draws of make_inputs (same generator order), each
    tensor quantized by quantize_e4m3.  Returns (q8, k8, v8, (q_s, k_s, v_s),
    kv_len) on the CPU."""
    q, k, v, kv_len = make_inputs(B, H, N, d, "f32", seed, padded, q_mul, kv_lo)
    (q8, qs), (k8, ks), (v8, vs) = (quantize_e4m3(t) for t in (q, k, v))
    return q8, k8, v8, (qs, ks, vs), kv_len
