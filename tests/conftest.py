import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # tests/test_sanitize_cpu.py runs CPU suites against a sanitized host build
    # of the library, named here; load_library() then returns that build
    lib = os.environ.get("PA_TEST_LIBRARY")
    if lib:
        import paged_kv_cache_64_amd as pa

        pa.load_library(lib)
