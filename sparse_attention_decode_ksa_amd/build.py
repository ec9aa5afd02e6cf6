"""Build libksa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m sparse_attention_decode_ksa_amd.build``; the repository's
``__graft_entry__.build()`` calls :func:`build_library` too.  Object files go to
``_build/`` at the repository root; the shared library is written next to this
file, where the Python binding loads it from.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libksa.so")
OBJDIR = os.path.join(ROOT, "_build", "ksa")
SOURCES = ["api.hip", "summaries.hip", "select.hip", "attention.hip", "vote.hip", "decode_step.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libksa)")


def compile_flags() -> list[str]:
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
        # packed-fp32 VALU forms are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I" + os.path.join(ROOT, "include"),
    ] + os.environ.get("KSA_EXTRA_FLAGS", "").split()


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-8000:]))
    return obj


def build_library(jobs: int | None = None, out: str | None = None, objdir: str | None = None) -> str:
    """Compile every source and link libksa.so (or `out`); returns its path.
    KSA_EXTRA_FLAGS adds hipcc flags (e.g. -D tuning macros for a variant build)."""
    global OBJDIR
    lib_out = out or LIB
    if objdir:
        OBJDIR = objdir
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = lib_out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-8000:]))
    os.replace(tmp, lib_out)
    return lib_out


PROBE_SOURCE = "read_probe.hip"
PROBE_LIB = os.path.join(PKG, "libksa_probe.so")


def build_probe(out: str | None = None) -> str:
    """Compile the measurement-only read probe (csrc/read_probe.hip) into
    libksa_probe.so, which bench.py --read-probe loads; it is not part of
    libksa.so or its header."""
    lib_out = out or PROBE_LIB
    tmp = lib_out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + compile_flags() + ["-shared", os.path.join(CSRC, PROBE_SOURCE), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (PROBE_SOURCE, " ".join(cmd), r.stderr[-8000:]))
    os.replace(tmp, lib_out)
    return lib_out


if __name__ == "__main__":
    print(build_library())
    print(build_probe())
    sys.exit(0)
