"""Build libq4k.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950."""

from __future__ import annotations

import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libq4k.so")
SOURCES = ["api.hip", "dequant.hip", "gemv.hip", "batched.hip", "prefill.hip"]
ARCH = os.environ.get("Q4K_OFFLOAD_ARCH", "gfx950")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 are generated anywhere.
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra", "-Wno-unused-parameter",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# batched.hip: matrix-core accumulators in ordinary vector registers.  The
# staged kernels otherwise keep some values in accumulation registers and
# copy them back before every use (about 1.3 copies per MFMA at 48 rows and
# 64 tokens); results are bitwise the same, 9B gate 64 tokens 31.4 -> 30.5 us.
SOURCE_FLAGS = {"batched.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False, out: str = LIB, extra_flags=()) -> str:
    """Compile every source (in parallel) and link libq4k.so in place.

    ``out`` and ``extra_flags`` (e.g. -D launch-shape macros) let a variant be
    built next to the default library for comparison."""
    objdir = os.path.join(HERE, "_build", hashlib.sha1(" ".join(extra_flags).encode()).hexdigest()[:8])
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = ["hipcc", *FLAGS, *SOURCE_FLAGS.get(src, []), *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        log, _ = p.communicate()
        text = log.decode(errors="replace")
        # the host pass does not know the device-only feature flag
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            print(f"[{src}]\n" + "\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = out + ".tmp"
    subprocess.check_call(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


STREAM_SRC = os.path.join(CSRC, "stream_read.hip")
STREAM_LIB = os.path.join(HERE, "libq4k_stream.so")


def build_stream_probe(verbose: bool = False, out: str = STREAM_LIB) -> str:
    """The read-only streaming kernel the benchmark reports as the device's
    achievable read rate (a library of its own, outside the q4k ABI)."""
    tmp = out + ".tmp"
    cmd = ["hipcc", *FLAGS, "-shared", STREAM_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    lines = [ln for ln in r.stdout.decode(errors="replace").splitlines() if "packed-fp32-ops" not in ln]
    if lines:
        print("[stream_read.hip]\n" + "\n".join(lines), file=sys.stderr)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for stream_read.hip")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_stream_probe(verbose=True))
