"""Thin Python binding of the attnio C ABI (argument marshalling only).

Every function here has the name of the C entry point it calls.  torch is used
only for device memory and the current HIP stream; every step of the attention
computation runs in the gfx950 kernels of libattnio.so.  There is no fallback:
if the library has not been built, the calls raise.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch  # imported first so that libattnio.so binds to torch's HIP runtime

# ATTNIO_LIB names another build of the same library (the LDS-poison debug
# build, for instance); it must exist, there is no fallback either way.
_LIB_PATH = os.environ.get("ATTNIO_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib",
                                                         "libattnio.so")
_lib = None

ATTN_OK = 0

__all__ = ["attn_fwd", "attn_fwd_f32", "attn_fwd_lse", "attn_fwd_f32_lse", "attn_bwd", "attn_bwd_noalloc",
           "attn_bwd_workspace_bytes", "attn_fwd_unfused", "attn_fwd_unfused_workspace_bytes",
           "stream_softmax", "stream_layernorm", "stream_rows_cached", "attn_fwd_fp8", "attn_strerror", "attn_version", "attn_query_tiling",
           "attn_tiling_count", "attn_tiling_get", "attn_tiling_enumerate", "attn_io_bound_bytes", "attn_fwd_tiled",
           "attn_io_model", "library_path", "load_library"]


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libattnio.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m exact_long_sequence_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    for name in ("attn_fwd", "attn_fwd_f32"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, vp]
        fn.restype = i32
    for name in ("attn_fwd_lse", "attn_fwd_f32_lse"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, vp]
        fn.restype = i32
    lib.attn_bwd.argtypes = [vp] * 10 + [i32, i32, i32, i32, f32, i32, vp, vp]
    lib.attn_bwd.restype = i32
    lib.attn_bwd_noalloc.argtypes = [vp] * 9 + [i32, i32, i32, i32, f32, i32, vp, vp]
    lib.attn_bwd_noalloc.restype = i32
    lib.attn_bwd_workspace_bytes.argtypes = [i32, i32, i32]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_fwd_unfused.argtypes = [vp] * 5 + [ctypes.c_size_t, i32, i32, i32, i32, f32, i32, vp, vp]
    lib.attn_fwd_unfused.restype = i32
    lib.attn_fwd_unfused_workspace_bytes.argtypes = [i32]
    lib.attn_fwd_unfused_workspace_bytes.restype = ctypes.c_size_t
    lib.stream_softmax.argtypes = [vp, vp, i32, i32, f32, vp]
    lib.stream_softmax.restype = i32
    lib.stream_layernorm.argtypes = [vp, vp, vp, vp, i32, i32, f32, vp]
    lib.stream_layernorm.restype = i32
    lib.stream_rows_cached.argtypes = [i32]
    lib.stream_rows_cached.restype = i32
    lib.attn_fwd_fp8.argtypes = [vp] * 4 + [i32] * 4 + [f32] * 4 + [i32, vp, vp]
    lib.attn_fwd_fp8.restype = i32
    lib.attn_strerror.argtypes = [i32]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = i32
    ip = ctypes.POINTER(ctypes.c_int)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.attn_query_tiling.argtypes = [i32, i32, i32, ip, ip, ip]
    lib.attn_query_tiling.restype = i32
    lib.attn_tiling_count.argtypes = []
    lib.attn_tiling_count.restype = i32
    lib.attn_tiling_get.argtypes = [i32, vp]
    lib.attn_tiling_get.restype = i32
    lib.attn_tiling_enumerate.argtypes = [i32, i32, i32, vp, i32]
    lib.attn_tiling_enumerate.restype = i32
    lib.attn_io_bound_bytes.argtypes = [i32, i32, i32, i32, i32, i32, vp, dp, dp, dp]
    lib.attn_io_bound_bytes.restype = i32
    lib.attn_fwd_tiled.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, i32, vp]
    lib.attn_fwd_tiled.restype = i32
    lib.attn_io_model.argtypes = [i32, i32, i32, i32, i32, i32, vp, ctypes.POINTER(ctypes.c_double)]
    lib.attn_io_model.restype = i32
    _lib = lib
    return lib


def attn_strerror(code: int) -> str:
    return load_library().attn_strerror(int(code)).decode()


def attn_version() -> int:
    return int(load_library().attn_version())


_DTYPES = {"bf16": 0, "f32": 1, "fp8": 2}


class AttnTiling(ctypes.Structure):
    """attn_tiling of include/attnio.h."""
    _fields_ = [(n, ctypes.c_int) for n in ("d", "BM", "BN", "stages", "waves", "lds_bytes", "wg_per_cu",
                                            "qb", "pingpong", "rowsum_mfma", "rowsum_in_stream", "mfma16")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class AttnTilingEval(ctypes.Structure):
    """attn_tiling_eval of include/attnio.h."""
    _fields_ = [("t", AttnTiling), ("compiled", ctypes.c_int), ("vgpr_estimate", ctypes.c_int),
                ("vgpr_budget", ctypes.c_int)] + \
               [(n, ctypes.c_double) for n in ("mfma_cycles", "valu_cycles", "issue_cycles_per_pair",
                                               "lds_read_bytes_per_pair", "l2_to_lds_bytes_per_pair",
                                               "beyond_l2_bytes_per_pair", "cycles_per_pair")] + \
               [("bound", ctypes.c_int)]

    def as_dict(self) -> dict:
        d = {n: getattr(self, n) for n, _ in self._fields_ if n != "t"}
        d["tiling"] = self.t.as_dict()
        return d


def attn_query_tiling(d: int, causal: bool = False, dtype: str = "bf16") -> dict:
    """(BM, BN, stages) of the tiling the path of `dtype` uses for head size d."""
    lib = load_library()
    vals = [ctypes.c_int(0) for _ in range(3)]
    rc = lib.attn_query_tiling(int(d), _DTYPES[dtype], int(bool(causal)), *[ctypes.byref(x) for x in vals])
    if rc != ATTN_OK:
        raise RuntimeError(attn_strerror(rc))
    return dict(zip(("BM", "BN", "stages"), (x.value for x in vals)))


def attn_tiling_count() -> int:
    return int(load_library().attn_tiling_count())


def attn_tiling_get(index: int) -> dict:
    t = AttnTiling()
    rc = load_library().attn_tiling_get(int(index), ctypes.byref(t))
    if rc != ATTN_OK:
        raise RuntimeError(attn_strerror(rc))
    return t.as_dict()


def attn_tiling_enumerate(d: int, causal: bool = False, dtype: str = "bf16", max_out: int = 256) -> list:
    """The model's feasible tilings for head size d, best first (list of dicts)."""
    arr = (AttnTilingEval * max_out)()
    n = load_library().attn_tiling_enumerate(int(d), _DTYPES[dtype], int(bool(causal)), arr, int(max_out))
    if n < 0:
        raise RuntimeError(attn_strerror(n))
    return [arr[i].as_dict() for i in range(min(n, max_out))]


def attn_io_bound_bytes(B: int, H: int, N: int, d: int, causal: bool, dtype: str = "bf16",
                        kv_len_host=None) -> dict:
    """T_min, T_LDS and T_L2 of one call (bytes; see include/attnio.h)."""
    lib = load_library()
    out = [ctypes.c_double(0) for _ in range(3)]
    kv_ptr = None
    if kv_len_host is not None:
        arr = (ctypes.c_int32 * B)(*[int(x) for x in kv_len_host])
        kv_ptr = ctypes.cast(arr, ctypes.c_void_p)
    rc = lib.attn_io_bound_bytes(B, H, N, d, _DTYPES[dtype], int(bool(causal)), kv_ptr,
                                 *[ctypes.byref(x) for x in out])
    if rc != ATTN_OK:
        raise RuntimeError(attn_strerror(rc))
    return dict(zip(("t_min", "t_lds", "t_l2"), (x.value for x in out)))


def attn_fwd_tiled(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tiling_index: int, *,
                   causal: bool = False, kv_len: Optional[torch.Tensor] = None,
                   scale: Optional[float] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """attn_fwd with the compiled tiling attn_tiling_get(tiling_index)."""
    lib = load_library()
    _check(q, k, v, torch.bfloat16)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    kv_len, kv_ptr = _kv_len_ptr(kv_len, B, q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.attn_fwd_tiled(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, d,
                                float(scale), int(bool(causal)), kv_ptr, int(tiling_index), stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"attn_fwd_tiled: {attn_strerror(rc)} (code {rc})")
    return out


def attn_io_model(B: int, H: int, N: int, d: int, elem_bytes: int, causal: bool,
                  kv_len_host=None) -> dict:
    """Host-side I/O model of one call (see include/attnio.h)."""
    lib = load_library()
    out = (ctypes.c_double * 5)()
    kv_ptr = None
    if kv_len_host is not None:
        arr = (ctypes.c_int32 * B)(*[int(x) for x in kv_len_host])
        kv_ptr = ctypes.cast(arr, ctypes.c_void_p)
    rc = lib.attn_io_model(B, H, N, d, elem_bytes, int(bool(causal)), kv_ptr, out)
    if rc != ATTN_OK:
        raise RuntimeError(attn_strerror(rc))
    return dict(zip(("t_min", "t_lds", "t_l2", "flops", "pairs"), list(out)))


def _check(q, k, v, dtype):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device, got {t.device}")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, H, N, d]")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, d], got {tuple(t.shape)}")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")


def _kv_len_ptr(kv_len, B, device):
    """Returns (tensor kept alive, device pointer or None)."""
    if kv_len is None:
        return None, None
    if not isinstance(kv_len, torch.Tensor):
        kv_len = torch.tensor(kv_len, dtype=torch.int32)
    if kv_len.device != device or kv_len.dtype != torch.int32:
        kv_len = kv_len.to(device=device, dtype=torch.int32)
    kv_len = kv_len.contiguous()
    if kv_len.numel() != B:
        raise ValueError(f"kv_len must have B={B} entries, got {kv_len.numel()}")
    return kv_len, kv_len.data_ptr()


def _call(fn_name, dtype, q, k, v, causal, kv_len, scale, out, lse=False):
    lib = load_library()
    _check(q, k, v, dtype)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    lse_t = None
    if lse is not False:
        if lse is None or lse is True:
            lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        else:
            lse_t = lse
            if (lse_t.shape != (B, H, N) or lse_t.dtype != torch.float32 or not lse_t.is_contiguous()
                    or lse_t.device != q.device):
                raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    kv_len, kv_ptr = _kv_len_ptr(kv_len, B, q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        ptrs = [q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()]
        if lse_t is not None:
            ptrs.append(lse_t.data_ptr())
        rc = getattr(lib, fn_name)(*ptrs, B, H, N, d, float(scale), int(bool(causal)), kv_ptr, stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"{fn_name}: {attn_strerror(rc)} (code {rc})")
    return out if lse_t is None else (out, lse_t)


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
             kv_len: Optional[torch.Tensor] = None, scale: Optional[float] = None,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 exact attention forward on [B, H, N, d] device tensors (d in {64, 128}).

    kv_len: None or int32 [B] key-padding lengths (moved to the device if needed).
    scale: defaults to 1/sqrt(d).  Enqueued on the current stream; no synchronisation."""
    return _call("attn_fwd", torch.bfloat16, q, k, v, causal, kv_len, scale, out)


def attn_fwd_f32(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                 kv_len: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 exact attention forward; same contract as attn_fwd."""
    return _call("attn_fwd_f32", torch.float32, q, k, v, causal, kv_len, scale, out)


def attn_fwd_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                 kv_len: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """bf16 forward that also returns the per-row log-sum-exp (float32 [B, H, N],
    -inf for rows without a visible key).  Returns (out, lse)."""
    return _call("attn_fwd_lse", torch.bfloat16, q, k, v, causal, kv_len, scale, out,
                 lse if lse is not None else None)


def attn_fwd_f32_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                     kv_len: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """fp32 forward with the log-sum-exp side output; returns (out, lse)."""
    return _call("attn_fwd_f32_lse", torch.float32, q, k, v, causal, kv_len, scale, out,
                 lse if lse is not None else None)


def attn_bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    """Device workspace bytes attn_bwd needs (0 for non-positive sizes)."""
    return int(load_library().attn_bwd_workspace_bytes(int(B), int(H), int(N)))


def attn_bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                     dout: torch.Tensor, lse: torch.Tensor, *, causal: bool = False,
                     kv_len: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                     dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                     dv: Optional[torch.Tensor] = None):
    """attn_bwd without a workspace: the library's static device scratch holds
    the row statistics (at most ATTN_NOALLOC_SCRATCH_BYTES).  Pass dq, dk, dv
    to make the call itself allocate nothing.  Returns (dq, dk, dv)."""
    lib = load_library()
    _check(q, k, v, torch.bfloat16)
    _check(o, dout, q, torch.bfloat16)
    B, H, N, d = q.shape
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must have q's shape")
    if (not isinstance(lse, torch.Tensor) or lse.shape != (B, H, N) or lse.dtype != torch.float32
            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    grads = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty_like(q)
        elif t.shape != q.shape or t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous bf16 tensor like q")
        grads.append(t)
    kv_len, kv_ptr = _kv_len_ptr(kv_len, B, q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  dout.data_ptr(), lse.data_ptr(), grads[0].data_ptr(),
                                  grads[1].data_ptr(), grads[2].data_ptr(), B, H, N, d, float(scale),
                                  int(bool(causal)), kv_ptr, stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"attn_bwd_noalloc: {attn_strerror(rc)} (code {rc})")
    return tuple(grads)


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
             dout: torch.Tensor, lse: torch.Tensor, *, causal: bool = False,
             kv_len: Optional[torch.Tensor] = None, scale: Optional[float] = None,
             dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
             dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """bf16 attention backward from the forward's (q, k, v, o, lse) and dout.

    causal, kv_len and scale must be those of the forward that produced o and
    lse.  Returns (dq, dk, dv).  workspace: optional uint8 device tensor of at
    least attn_bwd_workspace_bytes(B, H, N) bytes."""
    lib = load_library()
    _check(q, k, v, torch.bfloat16)
    _check(o, dout, q, torch.bfloat16)
    B, H, N, d = q.shape
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must have q's shape")
    if (not isinstance(lse, torch.Tensor) or lse.shape != (B, H, N) or lse.dtype != torch.float32
            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    grads = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty_like(q)
        elif t.shape != q.shape or t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous bf16 tensor like q")
        grads.append(t)
    need = attn_bwd_workspace_bytes(B, H, N)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif (workspace.device != q.device or not workspace.is_contiguous()
          or workspace.numel() * workspace.element_size() < need):
        raise ValueError(f"workspace must be a contiguous device buffer of >= {need} bytes")
    kv_len, kv_ptr = _kv_len_ptr(kv_len, B, q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                          lse.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(),
                          grads[2].data_ptr(), workspace.data_ptr(), B, H, N, d, float(scale),
                          int(bool(causal)), kv_ptr, stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"attn_bwd: {attn_strerror(rc)} (code {rc})")
    return tuple(grads)


def attn_fwd_unfused_workspace_bytes(N: int) -> int:
    """Workspace bytes one head of the unfused forward needs (6 N^2)."""
    return int(load_library().attn_fwd_unfused_workspace_bytes(int(N)))


def attn_fwd_unfused(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                     kv_len: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     heads_per_pass: int = 1) -> torch.Tensor:
    """Operator-centric bf16 forward (scores, softmax, P V as three kernels with
    the N x N intermediates in a workspace).  Same contract as attn_fwd.

    workspace: optional uint8 device tensor; by default one of
    heads_per_pass * attn_fwd_unfused_workspace_bytes(N) bytes is allocated."""
    lib = load_library()
    _check(q, k, v, torch.bfloat16)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous bf16 tensor like q")
    if workspace is None:
        per_head = attn_fwd_unfused_workspace_bytes(N)
        workspace = torch.empty(per_head * max(1, int(heads_per_pass)), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device buffer")
    ws_bytes = workspace.numel() * workspace.element_size()
    kv_len, kv_ptr = _kv_len_ptr(kv_len, B, q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.attn_fwd_unfused(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  workspace.data_ptr(), ws_bytes, B, H, N, d, float(scale),
                                  int(bool(causal)), kv_ptr, stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"attn_fwd_unfused: {attn_strerror(rc)} (code {rc})")
    return out


def stream_rows_cached(N: int) -> bool:
    """True if a row of N elements is held in registers (read from HBM once)."""
    return bool(load_library().stream_rows_cached(int(N)))


def _check_rows(x, out):
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or x.dtype != torch.bfloat16:
        raise TypeError("x must be a bf16 tensor on a GPU device")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [R, N] tensor")
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous bf16 tensor like x")
    return out


def stream_softmax(x: torch.Tensor, scale: float = 1.0, *, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Row softmax of scale * x for a bf16 [R, N] device tensor (out may be x)."""
    lib = load_library()
    out = _check_rows(x, out)
    R, N = x.shape
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = lib.stream_softmax(x.data_ptr(), out.data_ptr(), R, N, float(scale), stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"stream_softmax: {attn_strerror(rc)} (code {rc})")
    return out


def stream_layernorm(x: torch.Tensor, gamma: Optional[torch.Tensor] = None,
                     beta: Optional[torch.Tensor] = None, eps: float = 1e-5, *,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Row LayerNorm of a bf16 [R, N] device tensor; gamma / beta bf16 [N] or None."""
    lib = load_library()
    out = _check_rows(x, out)
    R, N = x.shape
    ptrs = []
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is None:
            ptrs.append(None)
            continue
        if (not isinstance(t, torch.Tensor) or t.device != x.device or t.dtype != torch.bfloat16
                or t.numel() != N or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous bf16 tensor of N={N} elements on x's device")
        ptrs.append(t.data_ptr())
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = lib.stream_layernorm(x.data_ptr(), ptrs[0], ptrs[1], out.data_ptr(), R, N, float(eps), stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"stream_layernorm: {attn_strerror(rc)} (code {rc})")
    return out


def attn_fwd_fp8(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, descale, *,
                 causal: bool = False, kv_len: Optional[torch.Tensor] = None,
                 scale: Optional[float] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp8 (OCP E4M3) attention forward: q8, k8, v8 are uint8 (or float8_e4m3fn)
    [B, H, N, d] device tensors, descale = (q_s, k_s, v_s) with x = fp8 * s.
    Returns bf16 [B, H, N, d]."""
    lib = load_library()
    ts = []
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise TypeError(f"{name} must be a GPU tensor")
        if t.dtype not in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
            raise TypeError(f"{name} must hold E4M3 bytes (uint8 or float8_e4m3fn), got {t.dtype}")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
        ts.append(t)
    if not (q8.shape == k8.shape == v8.shape) or not (q8.device == k8.device == v8.device):
        raise ValueError("q8, k8, v8 must share one shape and device")
    B, H, N, d = q8.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    elif out.shape != q8.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != q8.device:
        raise ValueError("out must be a contiguous bf16 tensor of q8's shape")
    qs, ks, vs = (float(x) for x in descale)
    kv_len, kv_ptr = _kv_len_ptr(kv_len, B, q8.device)
    with torch.cuda.device(q8.device):
        stream = torch.cuda.current_stream(q8.device).cuda_stream
        rc = lib.attn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(), B, H, N, d,
                              float(scale), qs, ks, vs, int(bool(causal)), kv_ptr, stream)
    if rc != ATTN_OK:
        raise RuntimeError(f"attn_fwd_fp8: {attn_strerror(rc)} (code {rc})")
    return out
