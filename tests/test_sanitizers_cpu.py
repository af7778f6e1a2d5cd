"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

libq4k's sources are compiled with the sanitizers on the host side only (the
device code is unchanged), linked with tests/sanitizer_driver.cpp, and the
driver runs every entry point's validation path with fake device addresses:
no GPU is used.  A sanitizer report or a wrong status fails the test.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")

SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LINK = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def test_abi_validation_under_sanitizers(tmp_path):
    from q4_dequant_gemv_amd import build as hip_build

    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    clangxx = os.path.join(rocm, "llvm", "bin", "clang++")
    if not os.path.exists(clangxx):
        pytest.skip("ROCm clang++ not found")
    objs = []
    procs = []
    for src in hip_build.SOURCES:
        obj = str(tmp_path / (src + ".o"))
        objs.append(obj)
        cmd = ["hipcc", *hip_build.FLAGS, "-O1", "-g", *SAN_HOST, "-c", os.path.join(hip_build.CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        assert p.returncode == 0, f"{src}: {out[-2000:]}"
    drv = str(tmp_path / "driver.o")
    subprocess.check_call([clangxx, "-O1", "-g", *SAN_LINK, "-I", os.path.join(ROOT, "include"), "-c",
                           os.path.join(ROOT, "tests", "sanitizer_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "driver")
    subprocess.check_call([clangxx, *SAN_LINK, drv, *objs, "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", exe])
    env = dict(os.environ)
    # the HIP runtime keeps allocations until exit: leaks are not what is checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, f"driver failed ({r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
