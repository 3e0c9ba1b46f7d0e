"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The front end (argument checks, device check, tiling model, I/O model) is
compiled with both sanitizers on its host code only (-Xarch_host before each
-fsanitize=, so no device code is instrumented), linked with the ordinary
kernel objects into a small driver (tests/sanitize/abi_driver.cpp) that calls
every entry point with arguments its checks must refuse and the host-only
queries over their ranges.  No GPU is needed: calls that pass the checks stop
at the device check.  Any sanitizer report or failed expectation fails the
test.
"""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_long_sequence_amd", "csrc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    from exact_long_sequence_amd import build
    try:
        return build.hipcc(), build
    except RuntimeError:
        return None, build


def test_host_code_is_clean_under_asan_and_ubsan():
    cc, build = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    host_tus = {"attnio_api.hip", "tile_model.cpp"}
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="attnio_san_") as tmp:
        objs, procs = [], []
        for src in build.SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            extra = SAN if src in host_tus else []
            cmd = [cc, *build.HIPCC_FLAGS, *build.FILE_FLAGS.get(src, []), *extra, *inc, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        for p in procs:
            out, _ = p.communicate()
            assert p.returncode == 0, out[-3000:]
        exe = os.path.join(tmp, "abi_driver")
        drv = os.path.join(tmp, "abi_driver.o")
        for cmd in ([cc, *build.HIPCC_FLAGS, *SAN, *inc, "-c",
                     os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", drv],
                    [cc, *build.HIPCC_FLAGS, *SAN, drv, *objs, "-o", exe]):
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        text = r.stdout + r.stderr
        assert "AddressSanitizer" not in text and "runtime error:" not in text, text[-4000:]
        assert r.returncode == 0 and "all checks passed" in r.stdout, text[-4000:]
