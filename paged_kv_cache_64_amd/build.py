"""Compiles the HIP library (libpa.so) for gfx950 with hipcc, in-tree."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
PROBE_LIB = os.path.join(HERE, "libpa_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are kept out of generated code on purpose.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = [os.path.join(CSRC, "pa_api.cpp"), os.path.join(CSRC, "pa_kernels.hip")]
    _run([HIPCC] + COMMON + inc + ["-o", LIB + ".tmp"] + srcs, verbose)
    os.replace(LIB + ".tmp", LIB)
    _run([HIPCC] + COMMON + inc + ["-o", PROBE_LIB + ".tmp", os.path.join(CSRC, "pa_probe.hip")],
         verbose)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
