"""The gfx950 FP8 conversions the FP8 kernels use, against the oracle's
E4M3 decoder and encoder (bit-exact)."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "paged_kv_cache_64_amd", "libpa_probe.so")


def _lib():
    lib = ctypes.CDLL(LIB)
    lib.pa_probe_fp8_decode.argtypes = [ctypes.c_void_p] * 3
    lib.pa_probe_fp8_decode.restype = ctypes.c_int32
    lib.pa_probe_fp8_decode_f16.argtypes = [ctypes.c_void_p] * 3
    lib.pa_probe_fp8_decode_f16.restype = ctypes.c_int32
    lib.pa_probe_fp8_encode.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.pa_probe_fp8_encode.restype = ctypes.c_int32
    return lib


def test_hardware_fp8_decode_is_ocp_e4m3():
    lib = _lib()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    out = torch.empty(256, dtype=torch.float32, device="cuda")
    assert lib.pa_probe_fp8_decode(codes.data_ptr(), out.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_hardware_fp8_to_f16_pairs_are_exact():
    """The direct code -> F16 conversion (scale 1) the FP8 decode kernel uses:
    every finite code maps to its exact value, NaN codes to NaN."""
    lib = _lib()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    out = torch.empty(256, dtype=torch.float16, device="cuda")
    assert lib.pa_probe_fp8_decode_f16(codes.data_ptr(), out.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    zero = np.flatnonzero(want == 0)          # +0 and -0 keep their sign
    assert np.array_equal(np.signbit(got[zero]), np.signbit(want[zero]))


@pytest.mark.parametrize("scale", [1.0, 0.5, 3.0, 1.0 / 64])
def test_hardware_fp8_encode_matches_oracle_on_every_f16(scale):
    lib = _lib()
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    x = x[np.isfinite(x)]
    xd = torch.from_numpy(x.copy()).cuda()
    out = torch.empty(x.shape[0], dtype=torch.uint8, device="cuda")
    inv = float(np.float32(1.0 / scale))
    assert lib.pa_probe_fp8_encode(xd.data_ptr(), x.shape[0], inv, out.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.quantize_e4m3(x, scale))
