"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The plan builders and argument checks of pa_api.cpp do 64-bit record and slot
arithmetic over host arrays, and the oracle walks tables and caches by hand.
This test builds both with gcc's -fsanitize=address,undefined (the kernel
launchers replaced by stand-ins that launch nothing, tests/sanitize/) and runs
the plan, ABI and oracle-pin tests against those builds in a child process
with the ASan runtime preloaded; any report fails the run.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_64_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
       "-g", "-O1"]
SUITES = ["tests/test_plan_cpu.py", "tests/test_abi_cpu.py", "tests/test_oracle_pins.py",
          "tests/test_oracle_prefill.py", "tests/test_oracle_fp8.py"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def build_host_sanitized(out_dir):
    """libpa_host_san.so: pa_api.cpp + launcher stand-ins, sanitized.  It carries
    the same source hash as libpa.so (same sources), so the binding accepts it."""
    from paged_kv_cache_64_amd import build

    lib = os.path.join(out_dir, "libpa_host_san.so")
    cmd = (["g++", "-std=c++17", "-fPIC", "-shared", "-Wall", "-D__HIP_PLATFORM_AMD__",
            "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            f'-DPA_SOURCE_SHA256="{build.source_hash()}"'] + SAN +
           [os.path.join(CSRC, "pa_api.cpp"), os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
            "-o", lib])
    subprocess.run(cmd, check=True)
    return lib


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's ASan runtime is not installed")
def test_host_code_and_oracle_under_asan_and_ubsan(tmp_path):
    from oracle import build as obuild

    host = build_host_sanitized(str(tmp_path))
    orc = obuild.build(lib=str(tmp_path / "liboracle_san.so"), extra_flags=SAN)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": _runtime("libasan.so"),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PA_TEST_LIBRARY": host,
        "PA_ORACLE_LIB": orc,
        "OMP_NUM_THREADS": "4",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
                       + SUITES, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    report = r.stderr
    for mark in ("ERROR: AddressSanitizer", "runtime error:"):
        if mark in report:
            report = report[report.index(mark):]
            break
    tail = r.stdout[-2000:] + "\n" + report[:6000]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's ASan runtime is not installed")
def test_the_sanitized_run_catches_a_planted_overflow(tmp_path):
    """The same build and child process with one slip planted in a copy of
    pa_api.cpp: the plan builder's buffer-size check lets a plan 8 bytes too
    big through, so it writes past the caller's buffer.  ASan must stop the
    child at that write, which shows the run above really is sanitized."""
    from paged_kv_cache_64_amd import build

    src = open(os.path.join(CSRC, "pa_api.cpp")).read()
    anchor = "if (plan_host_bytes < inf.plan_bytes) return PA_ERR_WORKSPACE;"
    assert src.count(anchor) == 2
    bad = tmp_path / "pa_api_planted.cpp"
    bad.write_text(src.replace(anchor, "if (plan_host_bytes + 8 < inf.plan_bytes) return PA_ERR_WORKSPACE;", 1))
    lib = str(tmp_path / "libpa_planted.so")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    f'-DPA_SOURCE_SHA256="{build.source_hash()}"'] + SAN +
                   [str(bad), os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), "-o", lib], check=True)
    script = (
        "import ctypes, numpy as np\n"
        "import paged_kv_cache_64_amd as pa\n"
        f"lib = pa.load_library({lib!r})\n"
        "h = pa.pa_pool_create(pa.PoolDesc(1, 64, 16, 8, 128, pa.PA_F16), 1 << 20, 1 << 20)\n"
        "lens = np.array([100, 7, 3000], np.int32)\n"
        "info = pa.PlanInfo()\n"
        "assert lib.pa_decode_plan(h, lens.ctypes.data, 3, 32, None, 0, ctypes.byref(info)) == 0\n"
        "buf = np.empty(info.plan_bytes // 4 - 1, np.int32)\n"
        "print('calling', flush=True)\n"
        "lib.pa_decode_plan(h, lens.ctypes.data, 3, 32, buf.ctypes.data, buf.nbytes, ctypes.byref(info))\n"
        "print('not caught', flush=True)\n")
    env = dict(os.environ)
    env.update({"LD_PRELOAD": _runtime("libasan.so"), "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1"})
    r = subprocess.run([sys.executable, "-c", script], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert "calling" in r.stdout, r.stdout + r.stderr[-3000:]
    assert "not caught" not in r.stdout
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-3000:]
