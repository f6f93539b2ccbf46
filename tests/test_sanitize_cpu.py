"""Host sanitizer runs (AddressSanitizer + UndefinedBehaviorSanitizer) on the CPU.

The CPU oracle (oracle/oracle.c) is built with gcc and both sanitizers and driven through
every entry point on tiny inputs (tests/sanitize/oracle_driver.c).  The C ABI's host code
(mosaic_abi.cpp: validation, chunk and size helpers) is built with hipcc, the sanitizers
on its host side only, linked against launcher stand-ins, and driven through every entry
point's validation, the int64 edges and the empty problems (tests/sanitize/abi_driver.cpp).
Any sanitizer report fails the run.  No GPU is used.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", exe,
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm"])
    assert "oracle sanitizer driver ok" in _run([exe], env=ENV)


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    hipcc = _hipcc()
    inc = ["-I", os.path.join(ROOT, "include")]
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = ["-O1", "-g", "-std=c++20", *inc, *host_san]
    objs = []
    for src, extra in ((os.path.join(ROOT, "mask_only_logits_amd", "csrc", "mosaic_abi.cpp"),
                        ["-x", "hip", "--offload-arch=gfx950"]),
                       (os.path.join(SAN, "launch_stubs.cpp"), []),
                       (os.path.join(SAN, "abi_driver.cpp"), [])):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([hipcc, *extra, *flags, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    _run([hipcc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", "-o", exe, *objs])
    assert "abi sanitizer driver ok" in _run([exe], env=ENV)
