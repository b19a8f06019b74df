"""pa_decode_noalloc (partials in the library's fixed per-GPU array) against
pa_decode with a caller workspace, through the C ABI: two calls in a row, the
second with a smaller input, each equal bit for bit to pa_decode on the same
inputs (same kernels, same arithmetic) and within tolerance of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_64_amd as pa
import workloads
from tests.gpu_harness import Staged, compare, report

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_split_override(monkeypatch):
    monkeypatch.delenv("PA_SPLIT_TOKENS", raising=False)


def _both(st, lib):
    w = st.w
    q, tables = st.dev[0]
    lens = st.lens
    width = int(tables.shape[1])
    stream = torch.cuda.current_stream().cuda_stream
    n_ws = lib.pa_decode_workspace_bytes(st.pool.handle, w.batch, 32, w.max_context_len)
    assert n_ws > 0, "the case must use a workspace (several splits per sequence)"
    ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
    ref_out = torch.empty_like(q)
    assert lib.pa_decode(st.pool.handle, 0, q.data_ptr(), ref_out.data_ptr(), tables.data_ptr(), width,
                         lens.data_ptr(), w.batch, 32, w.max_context_len, ctypes.c_float(w.scale),
                         ws.data_ptr(), n_ws, stream) == pa.PA_OK
    out = torch.full_like(q, float("nan"))
    assert lib.pa_decode_noalloc(st.pool.handle, 0, q.data_ptr(), out.data_ptr(), tables.data_ptr(), width,
                                 lens.data_ptr(), w.batch, 32, w.max_context_len, ctypes.c_float(w.scale),
                                 stream) == pa.PA_OK
    torch.cuda.synchronize()
    return out, ref_out, n_ws


def test_noalloc_decode_equals_the_workspace_decode_on_two_calls():
    lib = pa.load_library()
    cases = [workloads.custom([3000, 17, 1, 2048, 0, 777], seed=71),   # 12 splits of 256 tokens
             workloads.custom([1000, 33], seed=72)]                     # then a smaller one
    for i, w in enumerate(cases):
        st = Staged(w)
        out, ref_out, n_ws = _both(st, lib)
        report(f"noalloc call {i}", batch=w.batch, max_ctx=w.max_context_len, workspace=n_ws)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"call {i}: bits differ"
        compare(f"noalloc call {i} vs oracle", out, st.reference(0))
        st.close()
