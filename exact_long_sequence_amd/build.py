"""Builds the HIP library libattnio.so in-tree for gfx950 with hipcc.

Each translation unit is compiled to an object of its own (in parallel, into a
temporary directory), then the objects are linked into one shared library.

Usage:  python -m exact_long_sequence_amd.build [--debug-poison]
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libattnio.so")
POISON_LIB_PATH = os.path.join(LIB_DIR, "libattnio_poison.so")
SOURCES = ["attnio_api.hip", "tile_model.cpp", "attn_fwd_bf16.hip", "attn_fwd_f32.hip",
           "attn_bwd_bf16.hip", "attn_bwd_dq_bf16.hip", "attn_bwd_dkdv_pp_bf16.hip",
           "attn_unfused_bf16.hip", "stream_rows.hip",
           "attn_fwd_fp8.hip"]

# Packed fp32 VALU ops are disabled for every HIP translation unit; hipcc -O3
# would otherwise form v_pk_{add,mul,fma}_f32 from plain float code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Per-file options.  The dQ kernel consumes MFMA results on the VALU; asking
# the compiler for the VGPR form of MFMA keeps those results out of the
# accumulation registers and removes the register-to-register copies (measured
# faster; the dK/dV kernel, at the register limit, measured slower with it).
FILE_FLAGS = {
    "attn_bwd_dq_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd[:3])} ...")


def build(verbose: bool = False, debug_poison: bool = False) -> str:
    """Build libattnio.so; with debug_poison, the LDS-poison debug build
    libattnio_poison.so instead (every K/V ring buffer NaN-filled as soon as
    the ring protocol frees it; for checking that protocol, not for use)."""
    os.makedirs(LIB_DIR, exist_ok=True)
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include")]
    defs = ["-DATTNIO_DEBUG_POISON=1"] if debug_poison else []
    lib_path = POISON_LIB_PATH if debug_poison else LIB_PATH
    with tempfile.TemporaryDirectory(prefix="attnio_build_") as tmpdir:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            cmds.append([cc, *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), *defs, *inc, "-c",
                         os.path.join(CSRC, src), "-o", obj])
        workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = lib_path + ".tmp"
        _run([cc, *HIPCC_FLAGS, "-shared", *objs, "-o", tmp], verbose)
        os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True, debug_poison="--debug-poison" in sys.argv[1:]))
