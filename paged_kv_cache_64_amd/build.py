"""Compiles the HIP library (libpa.so) for gfx950 with hipcc, in-tree.

The library carries a sha256 of the sources and flags it was built from (the
string "pa-source-sha256:<hex>"), so a loader can tell a stale build from a
current one without loading it.
"""
import hashlib
import os
import re
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
SOURCES = [os.path.join(ROOT, "include", "pa.h"), os.path.join(CSRC, "pa_internal.h"),
           os.path.join(CSRC, "pa_api.cpp"), os.path.join(CSRC, "pa_kernels.hip")]
PROBE_SOURCES = [os.path.join(CSRC, "pa_probe.hip")]
_MARK = re.compile(rb"pa-source-sha256:([0-9a-f]{64})")


def source_hash(sources=SOURCES) -> str:
    """sha256 over the compile flags and the bytes of every source file."""
    h = hashlib.sha256(" ".join(COMMON).encode())
    for path in sources:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()


def built_hash(lib_path: str):
    """The source hash a built library carries, or None."""
    with open(lib_path, "rb") as f:
        m = _MARK.search(f.read())
    return m.group(1).decode() if m else None


def check_current(lib_path: str = LIB, sources=SOURCES) -> None:
    """Raises RuntimeError unless lib_path exists and was built from the current sources."""
    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} is missing: build it with __graft_entry__.build()")
    have, want = built_hash(lib_path), source_hash(sources)
    if have != want:
        raise RuntimeError(f"{lib_path} was built from other sources (carries {have}, sources are "
                           f"{want}): rebuild it with __graft_entry__.build()")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = [os.path.join(CSRC, "pa_api.cpp"), os.path.join(CSRC, "pa_kernels.hip")]
    tag = [f'-DPA_SOURCE_SHA256="{source_hash()}"']
    _run([HIPCC] + COMMON + inc + tag + ["-o", LIB + ".tmp"] + srcs, verbose)
    os.replace(LIB + ".tmp", LIB)
    ptag = [f'-DPA_SOURCE_SHA256="{source_hash(PROBE_SOURCES)}"']
    _run([HIPCC] + COMMON + inc + ptag + ["-o", PROBE_LIB + ".tmp"] + PROBE_SOURCES, verbose)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
