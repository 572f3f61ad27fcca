"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source is compiled as for the release library (device code for gfx950
unchanged) with the sanitizers on the host side only, linked with
``tests/host_sanitizer_driver.c`` and run on the CPU.  The driver takes every
entry point through its host-side paths that end before a kernel launch:
argument validation, refused sizes, missing workspaces and the size queries,
over the workloads' shapes and the extremes of the int32 arguments.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from moe_expert_layer_segment_amd import build  # noqa: E402

CLANG = "/opt/rocm/lib/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"


@pytest.mark.skipif(not os.path.exists(CLANG) or shutil.which(build.hipcc()) is None,
                    reason="ROCm clang / hipcc not available")
def test_host_code_under_asan_ubsan(tmp_path):
    flags = [f for f in build.common_flags() if f != "-O3"] + ["-O1", "-g"] + SAN

    def compile_one(src):
        out = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        _run([build.hipcc()] + lang + flags + ["-c", os.path.join(build.CSRC, src), "-o", out])
        return out

    with ThreadPoolExecutor(max_workers=min(8, len(build.SOURCES))) as ex:
        objs = list(ex.map(compile_one, build.SOURCES))
    drv = str(tmp_path / "driver.o")
    _run([CLANG, "-O1", "-g", "-I", build.INCLUDE, "-c",
          os.path.join(ROOT, "tests", "host_sanitizer_driver.c"), "-o", drv])
    exe = str(tmp_path / "driver")
    _run([CLANG + "++", "-fsanitize=address,undefined", drv] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all host checks passed" in res.stdout
