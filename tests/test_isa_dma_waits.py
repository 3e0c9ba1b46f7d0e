"""The streamed kernels' key loops carry no compiler-inserted wait on the
vector-memory counter.

K/V (and Q/dO) tiles reach LDS by direct-to-LDS loads issued as inline
assembly, and each loop waits for them explicitly (`s_waitcnt vmcnt(N)` in
inline assembly) only where a tile must have landed, with later tiles still
in flight.  The same hardware counter also counts every ordinary global load.
If a value loaded before the loop (say a Q fragment) is first used inside it,
the compiler puts its own `s_waitcnt vmcnt(...)` there, and that wait also
drains the tile loads in flight: the pipeline silently degrades to one tile
at a time.  The kernels prevent it by consuming such values in an empty asm
before the loop.

This test compiles every translation unit of the fused kernels to gfx950
assembly (the library's own flags), finds each loop (the span of a backward
branch) whose body issues `global_load_lds` and holds no smaller such loop
(the key loop, not a loop around a whole pass), and requires every `s_waitcnt` naming vmcnt in it to come from inline assembly
(between the `;;#ASMSTART` / `;;#ASMEND` markers the compiler writes around
it).  A register spill reload inside such a loop fails it too (its wait is the
compiler's).  Not covered: the unfused baseline, whose P x V loop reads P from
HBM with ordinary loads by design, and the one-wave dK/dV kernel, compiled
only to measure the two-group form against (the backward dispatches the
latter).  Host only: hipcc cross-compiles.
"""

import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

from exact_long_sequence_amd import build as B

# translation units whose kernels stream tiles by direct-to-LDS loads
# (attn_bwd_bf16.hip holds the one-wave dK/dV kernel, not covered, and the
# delta kernel, which streams nothing)
DMA_SOURCES = ["attn_fwd_bf16.hip", "attn_fwd_fp8.hip", "attn_bwd_dq_bf16.hip", "attn_bwd_dkdv_pp_bf16.hip"]

_KERNEL = re.compile(r"^(_Z\S+):")
_LABEL = re.compile(r"^(\.LBB\w+):")
_BRANCH = re.compile(r"\bs_(?:cbranch_\w+|branch)\s+(\.LBB\w+)")


def dma_loop_waits(asm: str, skip=()):
    """(loops with direct-to-LDS loads and no smaller such loop inside, [(kernel,
    line) of compiler vmcnt waits in them]); kernels whose name contains an
    entry of skip are not scanned."""
    lines = asm.split("\n")
    in_asm, state = [], False
    for line in lines:
        if "ASMSTART" in line:
            state = True
        in_asm.append(state)
        if "ASMEND" in line:
            state = False
    starts = [(i, m.group(1)) for i, line in enumerate(lines) if (m := _KERNEL.match(line))]
    n_loops, bad = 0, []
    for (s, name), (e, _) in zip(starts, starts[1:] + [(len(lines), None)]):
        if any(k in name for k in skip):
            continue
        labels = {}
        for i in range(s, e):
            m = _LABEL.match(lines[i])
            if m:
                labels[m.group(1)] = i
        loops = []
        for i in range(s, e):
            m = _BRANCH.search(lines[i])
            if m and m.group(1) in labels and labels[m.group(1)] < i:
                a = labels[m.group(1)]
                if any("global_load_lds" in lines[j] for j in range(a, i + 1)):
                    loops.append((a, i))
        for a, b in loops:
            if any(a <= a2 and b2 <= b and (a2, b2) != (a, b) for a2, b2 in loops):
                continue  # holds a smaller loop with direct-to-LDS loads
            body = range(a, b + 1)
            n_loops += 1
            bad += [(name, lines[j].strip()) for j in body
                    if "s_waitcnt" in lines[j] and "vmcnt(" in lines[j] and not in_asm[j]]
    return n_loops, bad


def test_scanner_tells_asm_waits_from_compiler_waits():
    """The parser on a hand-written listing: one loop with a DMA, an asm wait
    (allowed) and a compiler wait (reported); a loop without a DMA is ignored,
    and so is a loop around an inner one (its waits are outside the inner loop)."""
    asm = "\n".join([
        "_Zk:",
        ".LBB0_0:",
        "  global_load_dwordx4 v[8:11], v4, s[0:1]",
        "  s_waitcnt vmcnt(0)",
        ".LBB0_1:",
        ";;#ASMSTART",
        "s_mov_b32 m0, s0",
        "global_load_lds_dwordx4 v1, s[2:3]",
        ";;#ASMEND",
        ";;#ASMSTART",
        "s_waitcnt vmcnt(4)",
        ";;#ASMEND",
        "  s_waitcnt vmcnt(0) lgkmcnt(0)",
        "  s_cbranch_scc1 .LBB0_1",
        ".LBB0_2:",
        "  global_load_dwordx4 v[0:3], v4, s[0:1]",
        "  s_waitcnt vmcnt(0)",
        "  s_cbranch_scc1 .LBB0_2",
        "  s_cbranch_scc1 .LBB0_0",
        "  s_endpgm",
    ])
    n, bad = dma_loop_waits(asm)
    assert n == 1
    assert bad == [("_Zk", "s_waitcnt vmcnt(0) lgkmcnt(0)")]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _compile(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    cmd = [_hipcc(), *B.HIPCC_FLAGS, *B.FILE_FLAGS.get(src, []), "-I", os.path.join(B.ROOT, "include"),
           "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return src, open(out).read()


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_no_compiler_vmcnt_wait_in_dma_loops(tmp_path):
    assert set(DMA_SOURCES) <= set(B.SOURCES)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(DMA_SOURCES), os.cpu_count() or 1)) as ex:
        listings = list(ex.map(lambda s: _compile(s, str(tmp_path)), DMA_SOURCES))
    problems = []
    for src, asm in listings:
        n, bad = dma_loop_waits(asm)
        assert n > 0, f"{src}: no loop with direct-to-LDS loads found (scanner out of date?)"
        problems += [(src, k[:80], w) for k, w in bad]
    assert problems == [], "compiler-inserted vmcnt waits inside DMA loops:\n" + "\n".join(map(str, problems))
