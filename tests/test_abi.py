"""C-ABI checks that need no GPU: the library loads, exports every entry point
that include/attnio.h declares, and rejects bad arguments on the host before
any device call.  The I/O model is checked against its closed forms."""

import ctypes
import math
import os
import re

import pytest

from exact_long_sequence_amd import attnio

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnio.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*((?:attn|stream)_\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attnio.library_path()):
        pytest.fail("libattnio.so is not built (run python -m exact_long_sequence_amd.build)")
    return attnio.load_library()


def test_header_declares_the_boundary():
    names = set(declared_functions())
    assert {"attn_fwd", "attn_fwd_f32", "attn_fwd_lse", "attn_fwd_f32_lse", "attn_bwd",
            "attn_bwd_workspace_bytes", "attn_fwd_unfused", "attn_fwd_unfused_workspace_bytes",
            "stream_softmax", "stream_layernorm", "stream_rows_cached", "attn_fwd_fp8", "attn_strerror",
            "attn_version", "attn_bwd_noalloc", "attn_tiling_count", "attn_tiling_get", "attn_fwd_tiled",
            "attn_tiling_enumerate", "attn_io_bound_bytes",
            "attn_query_tiling", "attn_io_model"} <= names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in attnio.h but not exported"


def test_strerror_and_version(lib):
    assert attnio.attn_version() >= 100
    for code in range(0, -10, -1):
        s = attnio.attn_strerror(code)
        assert s and "unknown" not in s
    assert "unknown" in attnio.attn_strerror(-99)


def test_query_tiling(lib):
    for d in (64, 128):
        for causal in (False, True):
            t = attnio.attn_query_tiling(d, causal)
            assert t["BM"] % 32 == 0 and t["BN"] % 32 == 0 and t["stages"] >= 2
            # K and V stages of BN x d bf16 rows fit the 160 KiB LDS of a gfx950 CU
            assert t["stages"] * 2 * t["BN"] * d * 2 <= 160 * 1024
        # the fp32 and fp8 paths have one tiling each
        assert attnio.attn_query_tiling(d, False, "f32") == {"BM": 8, "BN": 64, "stages": 1}
        assert attnio.attn_query_tiling(d, True, "fp8") == {"BM": 128, "BN": 128, "stages": 2}
    with pytest.raises(RuntimeError):
        attnio.attn_query_tiling(96, False)
    # the raw call: NULL outputs allowed, bad dtype and head size refused
    assert lib.attn_query_tiling(128, 0, 1, None, None, None) == 0
    assert lib.attn_query_tiling(128, 7, 1, None, None, None) == -8
    assert lib.attn_query_tiling(80, 0, 1, None, None, None) == -2


def test_tiling_table_and_explicit_tiling_errors(lib):
    n = attnio.attn_tiling_count()
    assert n >= 2
    seen = set()
    for i in range(n):
        t = attnio.attn_tiling_get(i)
        assert t["BM"] == 32 * t["waves"] * t["qb"] and t["d"] in (64, 128)
        assert t["wg_per_cu"] * t["lds_bytes"] <= 160 * 1024
        key = tuple(sorted(t.items()))
        assert key not in seen
        seen.add(key)
    with pytest.raises(RuntimeError):
        attnio.attn_tiling_get(n)
    assert lib.attn_tiling_get(0, None) == -1

    def call(index, d=64):
        return lib.attn_fwd_tiled(0x1000, 0x2000000, 0x4000000, 0x6000000, 1, 1, 16, d,
                                  ctypes.c_float(0.125), 0, None, index, None)
    assert call(-1) == -8 and call(n) == -8
    wrong_d = next(i for i in range(n) if attnio.attn_tiling_get(i)["d"] != 64)
    assert call(wrong_d, d=64) == -8            # the tiling's head size must match
    assert lib.attn_fwd_tiled(None, 0x2000000, 0x4000000, 0x6000000, 1, 1, 16, 64,
                              ctypes.c_float(0.125), 0, None, 0, None) == -1
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        right_d = next(i for i in range(n) if attnio.attn_tiling_get(i)["d"] == 64)
        assert call(right_d) == -6


def test_io_bound_bytes_matches_closed_forms(lib):
    B, H, N, d = 2, 3, 1000, 128
    for dtype, e in (("bf16", 2), ("f32", 4), ("fp8", 1)):
        io = attnio.attn_io_bound_bytes(B, H, N, d, False, dtype)
        assert io["t_min"] == e * d * B * H * (2 * N + 2 * N)     # no kv_len: no kv_len bytes
        assert io["t_lds"] >= io["t_min"] and io["t_l2"] >= io["t_min"]
    p = attnio.attn_io_bound_bytes(2, 1, 64, 64, True, "bf16", [10, 64])
    assert p["t_min"] == 8 + 2 * 64 * (2 * 64 + 2 * 10) + 2 * 64 * (2 * 64 + 2 * 64)
    # bf16 figures are those of attn_io_model for the same call
    m = attnio.attn_io_model(B, H, N, d, 2, True)
    io = attnio.attn_io_bound_bytes(B, H, N, d, True)
    assert (io["t_min"], io["t_lds"], io["t_l2"]) == (m["t_min"], m["t_lds"], m["t_l2"])
    assert lib.attn_io_bound_bytes(1, 1, 16, 64, 0, 0, None, None, None, None) == 0
    assert lib.attn_io_bound_bytes(0, 1, 16, 64, 0, 0, None, None, None, None) == -3
    assert lib.attn_io_bound_bytes(1, 1, 16, 96, 0, 0, None, None, None, None) == -2
    assert lib.attn_io_bound_bytes(1, 1, 16, 64, 9, 0, None, None, None, None) == -8


def _call(lib, name, q=0x1000, k=0x2000000, v=0x4000000, o=0x6000000, B=1, H=1, N=16, d=64,
          scale=0.125, causal=0):
    fn = getattr(lib, name)
    return fn(q, k, v, o, B, H, N, d, ctypes.c_float(scale), causal, None, None)


@pytest.mark.parametrize("name", ["attn_fwd_lse", "attn_fwd_f32_lse"])
def test_lse_entry_argument_errors(lib, name):
    fn = getattr(lib, name)

    def call(lse, q=0x1000, o=0x6000000):
        return fn(q, 0x2000000, 0x4000000, o, lse, 1, 1, 16, 64, ctypes.c_float(0.125), 0, None, None)
    assert call(None) == -1                      # LSE is required here
    assert call(0x8000002) == -4                 # not 4-byte aligned
    assert call(0x1000 + 16) == -7               # LSE overlaps Q
    assert call(0x6000000 + 4) == -7             # LSE overlaps O
    assert call(0x8000000, q=None) == -1         # the usual checks still apply


def test_bwd_workspace_bytes(lib):
    # two fp32 row statistics per row, rows padded to 64 per head
    assert attnio.attn_bwd_workspace_bytes(1, 1, 1) == 2 * 64 * 4
    assert attnio.attn_bwd_workspace_bytes(2, 3, 130) == 2 * 6 * 192 * 4
    assert attnio.attn_bwd_workspace_bytes(0, 1, 1) == 0
    assert attnio.attn_bwd_workspace_bytes(1, 1, -5) == 0


def test_bwd_entry_argument_errors(lib):
    # tensors of B*H*N*d = 1*1*16*64 bf16 = 2 KiB, spaced 1 MiB apart
    base = {"Q": 0x100000, "K": 0x200000, "V": 0x300000, "O": 0x400000, "dO": 0x500000,
            "LSE": 0x600000, "dQ": 0x700000, "dK": 0x800000, "dV": 0x900000, "ws": 0xA00000}

    def call(d=64, N=16, **over):
        p = dict(base, **over)
        return lib.attn_bwd(p["Q"], p["K"], p["V"], p["O"], p["dO"], p["LSE"], p["dQ"], p["dK"],
                            p["dV"], p["ws"], 1, 1, N, d, ctypes.c_float(0.125), 0, None, None)
    for name in base:
        assert call(**{name: None}) == -1, name
    assert call(d=96) == -2
    assert call(N=0) == -3
    for name in ("Q", "K", "V", "O", "dO", "dQ", "dK", "dV", "ws"):
        assert call(**{name: base[name] + 8}) == -4, name
    assert call(LSE=base["LSE"] + 2) == -4
    assert call(dQ=base["Q"] + 1024) == -7           # output overlaps an input
    assert call(dK=base["dO"]) == -7
    assert call(dV=base["LSE"] + 16) == -7
    assert call(ws=base["dQ"] + 512) == -7           # workspace overlaps an output
    assert call(dK=base["dV"] + 1024) == -7          # outputs overlap each other
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        assert call() == -6


def test_bwd_noalloc_host_checks(lib):
    """The allocation-free backward checks its arguments like attn_bwd and
    refuses, on the host, shapes whose statistics exceed its static scratch."""
    base = {"Q": 0x100000, "K": 0x200000, "V": 0x300000, "O": 0x400000, "dO": 0x500000,
            "LSE": 0x600000, "dQ": 0x700000, "dK": 0x800000, "dV": 0x900000}

    def call(B=1, H=1, N=16, d=64, **over):
        p = dict(base, **over)
        return lib.attn_bwd_noalloc(p["Q"], p["K"], p["V"], p["O"], p["dO"], p["LSE"], p["dQ"],
                                    p["dK"], p["dV"], B, H, N, d, ctypes.c_float(0.125), 0, None, None)
    for name in base:
        assert call(**{name: None}) == -1, name
    assert call(d=96) == -2 and call(N=0) == -3
    assert call(dQ=base["Q"] + 1024) == -7
    # 4194304 padded rows of 8 bytes fill the 32 MiB scratch exactly; 64 more do not
    assert attnio.attn_bwd_workspace_bytes(1, 4096, 1024) == 32 * 1024 * 1024
    G = 1 << 30
    big = {k: (i + 1) * G for i, k in enumerate(base)}
    assert call(B=1, H=4097, N=1024, **big) == -9
    assert call(B=1, H=4097, N=1024, **dict(big, Q=None)) == -1   # pointer checks come first
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        assert call() == -6
        assert call(B=1, H=4096, N=1024, **big) == -6               # fits: reaches the device check


def test_unfused_entry_argument_errors(lib):
    assert attnio.attn_fwd_unfused_workspace_bytes(1000) == 6 * 1000 * 1000
    assert attnio.attn_fwd_unfused_workspace_bytes(0) == 0
    ws = 0x10000000
    need = 6 * 16 * 16

    def call(q=0x1000, o=0x6000000, w=ws, nbytes=need, d=64):
        return lib.attn_fwd_unfused(q, 0x2000000, 0x4000000, o, w, nbytes, 1, 1, 16, d,
                                    ctypes.c_float(0.125), 0, None, None)
    assert call(w=None) == -1
    assert call(q=None) == -1
    assert call(d=96) == -2
    assert call(w=ws + 16) == -4                   # workspace must be 256-byte aligned
    assert call(nbytes=need - 1) == -8             # less than one head
    assert call(w=0x6000000 - 256) == -7           # workspace overlaps O
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        assert call() == -6


def test_fp8_entry_argument_errors(lib):
    def call(q=0x100000, o=0x400000, d=64, N=16, scale=0.125, qs=1.0, ks=1.0, vs=1.0):
        return lib.attn_fwd_fp8(q, 0x200000, 0x300000, o, 1, 1, N, d, ctypes.c_float(scale),
                                ctypes.c_float(qs), ctypes.c_float(ks), ctypes.c_float(vs), 0, None, None)
    assert call(q=None) == -1 and call(o=None) == -1
    assert call(d=96) == -2 and call(N=0) == -3
    assert call(q=0x100008) == -4
    assert call(scale=float("nan")) == -8
    assert call(qs=0.0) == -8 and call(ks=-1.0) == -8 and call(vs=float("inf")) == -8
    # finite descales whose folded exponent multiplier overflows fp32
    assert call(qs=2.0 ** 100, ks=2.0 ** 100) == -8
    assert call(scale=-2.0 ** 120, qs=2.0 ** 10) == -8
    assert call(o=0x300000 - 1024) == -7       # 2 KiB of bf16 output reaches into V's 1 KiB
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        assert call() == -6


def test_stream_rows_argument_errors(lib):
    X, Y, G = 0x100000, 0x900000, 0x2000000

    def sm(x=X, y=Y, R=4, N=1024, scale=1.0):
        return lib.stream_softmax(x, y, R, N, ctypes.c_float(scale), None)

    def ln(x=X, g=G, b=None, y=Y, R=4, N=1024, eps=1e-5):
        return lib.stream_layernorm(x, g, b, y, R, N, ctypes.c_float(eps), None)
    assert sm(x=None) == -1 and ln(y=None) == -1
    assert sm(R=0) == -3 and ln(N=0) == -3
    assert sm(R=1 << 20, N=1 << 20) == -3                 # R * N >= 2^40
    assert sm(x=X + 8) == -4 and ln(g=G + 2) == -4
    assert sm(scale=0.0) == -8 and sm(scale=-1.0) == -8 and sm(scale=float("nan")) == -8
    assert ln(eps=0.0) == -8 and ln(eps=float("inf")) == -8
    assert sm(y=X + 16) == -7                              # partial overlap
    assert ln(g=Y + 64) == -7                              # gamma inside the output
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        assert sm(y=X) == -6                               # in place passes the host checks
        assert ln(b=G + 4096) == -6
    assert attnio.stream_rows_cached(65536) and attnio.stream_rows_cached(8)
    assert not attnio.stream_rows_cached(65544) and not attnio.stream_rows_cached(1001)


@pytest.mark.parametrize("name", ["attn_fwd", "attn_fwd_f32"])
def test_host_side_argument_errors(lib, name):
    assert _call(lib, name, q=None) == -1
    assert _call(lib, name, o=None) == -1
    assert _call(lib, name, d=96) == -2
    assert _call(lib, name, d=0) == -2
    assert _call(lib, name, N=0) == -3
    assert _call(lib, name, B=-1) == -3
    assert _call(lib, name, B=1 << 12, H=1 << 12, N=1 << 12, d=64) == -3  # >= 2^31 elements
    assert _call(lib, name, q=0x1008) == -4
    assert _call(lib, name, o=0x1000 + 64) == -7  # O overlaps Q
    assert _call(lib, name, scale=float("nan")) == -8
    assert _call(lib, name, scale=float("inf")) == -8


def test_no_gpu_reports_device_error(lib):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call(lib, "attn_fwd") == -6


def test_io_model_closed_forms():
    B, H, N, d = 1, 2, 1000, 128
    m = attnio.attn_io_model(B, H, N, d, 2, False)
    assert m["t_min"] == 2 * d * H * (2 * N + 2 * N)
    assert m["pairs"] == H * N * N
    assert m["flops"] == 4 * d * H * N * N
    c = attnio.attn_io_model(B, H, N, d, 2, True)
    assert c["pairs"] == H * N * (N + 1) // 2
    # key padding: K and V are read only up to kv_len; pairs = N * L (non-causal)
    p = attnio.attn_io_model(2, 1, 64, 64, 2, False, [10, 64])
    assert p["t_min"] == 8 + 2 * 64 * (2 * 64 + 2 * 10) + 2 * 64 * (2 * 64 + 2 * 64)
    assert p["pairs"] == 64 * 10 + 64 * 64
    # causal with padding: sum_i min(i + 1, L)
    cp = attnio.attn_io_model(1, 1, 100, 64, 2, True, [30])
    assert cp["pairs"] == sum(min(i + 1, 30) for i in range(100))
    # L2->LDS traffic shrinks with the resident tile and exceeds the compulsory bytes
    assert m["t_lds"] >= m["t_min"]
    t = attnio.attn_query_tiling(d)
    nqt = math.ceil(N / t["BM"])
    ntile = math.ceil(N / t["BN"])
    assert m["t_lds"] == H * nqt * (t["BM"] * d * 2 + 2 * ntile * t["BN"] * d * 2)
    with pytest.raises(RuntimeError):
        attnio.attn_io_model(1, 1, 10, 72, 2, False)


def test_io_model_l2_generations():
    """Causal 32 heads x 32768 x 128: 8192 resident rows per XCD give four
    generations needing 32K, 24K, 16K and 8K keys; each later one reuses 8192
    keys (4 MiB of K+V rows of 512 B) from the previous, so K/V are read for
    32K + 16K + 8K + 0 keys per head, and Q and O once: 1.375 x T_min."""
    H, N, d = 32, 32768, 128
    t = attnio.attn_query_tiling(d, True)
    assert t["BM"] == 256
    m = attnio.attn_io_model(1, H, N, d, 2, True)
    row = d * 2
    l2_keys = 4 * 1024 * 1024 // (2 * row)
    resident = 32 * 256  # one 256-row workgroup per CU, 32 CUs per XCD
    gens = [N - g * resident for g in range(N // resident)]
    kv_keys = gens[0] + sum(k - min(l2_keys, k) for k in gens[1:])
    want = H * (2 * row * N + 2 * row * kv_keys)
    assert m["t_l2"] == want
    assert abs(m["t_l2"] / m["t_min"] - 1.375) < 1e-3
    # non-causal: one generation per 8192 rows, no reuse across generations
    nc = attnio.attn_io_model(1, 16, 8192, d, 2, False)
    assert nc["t_l2"] == 16 * (2 * row * 8192 + 2 * row * 8192)
