"""Builds decode_step (a plain-C program using libksa through include/ksa.h)
with the host C compiler, linked to the in-tree libksa.so and the HIP runtime.
__graft_entry__.build() calls build(); tests/test_gpu_c_abi.py runs the binary."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "decode_step.c")
BIN = os.path.join(HERE, "decode_step")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for the C ABI check")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"), SRC,
           "-L" + os.path.join(ROOT, "sparse_attention_decode_ksa_amd"), "-lksa",
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../sparse_attention_decode_ksa_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", BIN]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("C ABI check failed to build:\n%s\n%s" % (" ".join(cmd), r.stderr))
    return BIN


if __name__ == "__main__":
    print(build())
