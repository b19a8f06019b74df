"""The MFMA operand/result lane layouts the kernels rely on, each checked with
one MFMA against a plain matrix product: 16x16x16 f16 (shared-prefix pieces)
and 16x16x32 f16 (decode QK^T, prefill)."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "paged_kv_cache_64_amd", "libpa_probe.so")


def test_mfma_16x16x16_f16_lane_layout():
    lib = ctypes.CDLL(LIB)
    lib.pa_probe_mfma_16x16x16.argtypes = [ctypes.c_void_p] * 4
    lib.pa_probe_mfma_16x16x16.restype = ctypes.c_int32
    rng = np.random.default_rng(0)
    a = rng.integers(-4, 5, (16, 16)).astype(np.float16)   # small integers: exact in fp32
    b = rng.integers(-4, 5, (16, 16)).astype(np.float16)
    ad, bd = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    dd = torch.zeros((16, 16), dtype=torch.float32, device="cuda")
    assert lib.pa_probe_mfma_16x16x16(ad.data_ptr(), bd.data_ptr(), dd.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    want = a.astype(np.float64) @ b.astype(np.float64)
    assert np.array_equal(dd.cpu().numpy().astype(np.float64), want)


def test_mfma_16x16x32_f16_lane_layout():
    lib = ctypes.CDLL(LIB)
    lib.pa_probe_mfma_16x16x32.argtypes = [ctypes.c_void_p] * 4
    lib.pa_probe_mfma_16x16x32.restype = ctypes.c_int32
    rng = np.random.default_rng(1)
    a = rng.integers(-4, 5, (16, 32)).astype(np.float16)   # small integers: exact in fp32
    b = rng.integers(-4, 5, (32, 16)).astype(np.float16)
    ad, bd = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    dd = torch.zeros((16, 16), dtype=torch.float32, device="cuda")
    assert lib.pa_probe_mfma_16x16x32(ad.data_ptr(), bd.data_ptr(), dd.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    want = a.astype(np.float64) @ b.astype(np.float64)
    assert np.array_equal(dd.cpu().numpy().astype(np.float64), want)
