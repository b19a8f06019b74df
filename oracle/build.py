"""Builds the oracle's shared library with gcc.

TEST INFRASTRUCTURE: the oracle is a checker, not the product.  The library
carries a sha256 of its source and flags ("pa-oracle-source-sha256:<hex>"), so
the loader can rebuild a library that was made from other sources.
"""
import hashlib
import os
import re
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
LIB = os.path.join(HERE, "libpa_oracle.so")
DEFAULT_LIB = LIB
FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra"]
_MARK = re.compile(rb"pa-oracle-source-sha256:([0-9a-f]{64})")


def source_hash(extra_flags=()) -> str:
    h = hashlib.sha256(" ".join(FLAGS + list(extra_flags)).encode())
    with open(SRC, "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def is_current(lib=LIB, extra_flags=()) -> bool:
    """True when lib exists and was built from the current source and flags."""
    if not os.path.exists(lib):
        return False
    with open(lib, "rb") as f:
        m = _MARK.search(f.read())
    return bool(m) and m.group(1).decode() == source_hash(extra_flags)


def build(verbose: bool = False, lib=LIB, extra_flags=()) -> str:
    """extra_flags (for example sanitizer options) are part of the recorded hash."""
    tag = f'-DPA_ORACLE_SOURCE_SHA256="{source_hash(extra_flags)}"'
    cmd = ["gcc"] + FLAGS + list(extra_flags) + [tag, "-o", lib + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
