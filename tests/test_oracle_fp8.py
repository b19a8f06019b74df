"""Pins for the oracle's FP8 (OCP E4M3) storage functions, each against
something other than the oracle: closed forms of the format, torch's
float8_e4m3fn (CPU), round trips, tie cases, and the pinned F16 decode."""
import math

import numpy as np
import pytest
import torch

import oracle


def test_decoder_closed_forms():
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for code, want in cases.items():
        got = oracle.e4m3_to_f64(code)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), hex(code)
    assert math.isnan(oracle.e4m3_to_f64(0x7F)) and math.isnan(oracle.e4m3_to_f64(0xFF))


def test_decoder_matches_torch_on_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_encoder_matches_torch_on_every_f16_in_range():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    keep = np.isfinite(x) & (np.abs(x.astype(np.float64)) <= 448.0)
    xs = x[keep]
    ref = torch.from_numpy(xs.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = oracle.quantize_e4m3(xs, 1.0)
    assert np.array_equal(ours, ref)


def test_encoder_round_trips_saturates_and_ties_to_even():
    for c in range(256):
        v = oracle.e4m3_to_f64(c)
        if not math.isnan(v):
            assert oracle.f64_to_e4m3(v) == c, hex(c)
    assert oracle.f64_to_e4m3(1.0625) == 0x38        # halfway 1.0 / 1.125 -> even
    assert oracle.f64_to_e4m3(1.1875) == 0x3A        # halfway 1.125 / 1.25 -> even
    assert oracle.f64_to_e4m3(1.07) == 0x39
    assert oracle.f64_to_e4m3(449.0) == 0x7E and oracle.f64_to_e4m3(-1e9) == 0xFE
    assert oracle.f64_to_e4m3(2.0 ** -10) == 0x00      # halfway 0 / 2^-9 -> even (zero)
    assert oracle.f64_to_e4m3(3 * 2.0 ** -10) == 0x02  # halfway 2^-9 / 2^-8 -> even
    v = oracle.e4m3_to_f64(oracle.f64_to_e4m3(float("nan")))
    assert math.isnan(v)


def test_quantize_uses_the_reciprocal_scale():
    x = np.array([1.0, 3.0, -0.7, 100.0, 300.0], np.float16)
    want = [oracle.f64_to_e4m3(2.0), oracle.f64_to_e4m3(6.0),
            oracle.f64_to_e4m3(float(np.float32(x[2]) * np.float32(2.0))),
            oracle.f64_to_e4m3(200.0), 0x7E]                # 600 saturates to 448
    assert list(oracle.quantize_e4m3(x, 0.5)) == want
    # a scale whose reciprocal is not exact in fp32: the product is rounded to fp32 first
    inv = np.float32(1.0 / 3.0)
    got = oracle.quantize_e4m3(np.array([1.5], np.float16), 3.0)[0]
    assert got == oracle.f64_to_e4m3(float(np.float32(1.5) * inv))


def test_fp8_decode_reduces_to_the_f16_decode_on_dequantised_values():
    """Codes x power-of-two scales are exact in F16, so the FP8 oracle must
    equal the pinned F16 oracle fed with the dequantised values."""
    rng = np.random.default_rng(7)
    hq, hkv, d, bs, nb = 8, 2, 16, 4, 16
    lens = np.array([1, 5, 9, 16], np.int32)
    kc = rng.integers(0, 256, (nb * bs, hkv, d)).astype(np.uint8)
    vc = rng.integers(0, 256, (nb * bs, hkv, d)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x10                   # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x10
    tables = rng.permutation(nb).reshape(4, 4).astype(np.int32)
    q = rng.standard_normal((4, hq, d)).astype(np.float16)
    ks, vs = 0.25, 2.0
    lut = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    kf = (lut[kc] * ks).astype(np.float16)
    vf = (lut[vc] * vs).astype(np.float16)
    assert np.array_equal(kf.astype(np.float64), lut[kc] * ks)   # exact in F16
    a = oracle.decode_e4m3(q, kc, vc, tables, lens, 0.3, bs, ks, vs)
    b = oracle.decode(q, kf, vf, tables, lens, 0.3, bs)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_fp8_prefill_reduces_to_the_f16_prefill_on_dequantised_values():
    """A chunked-prefill step over FP8 codes with power-of-two scales equals
    the pinned F16 prefill oracle fed with the dequantised values (chunks of
    0, 1 and several tokens, with and without history)."""
    rng = np.random.default_rng(8)
    hq, hkv, d, bs, nb = 8, 2, 16, 4, 32
    q_lens = [3, 1, 0, 7, 5]
    lens = np.array([3, 9, 6, 16, 12], np.int32)
    starts = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    kc = rng.integers(0, 256, (nb * bs, hkv, d)).astype(np.uint8)
    vc = rng.integers(0, 256, (nb * bs, hkv, d)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x21                   # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x21
    tables = rng.permutation(nb)[:20].reshape(5, 4).astype(np.int32)
    q = rng.standard_normal((int(starts[-1]), hq, d)).astype(np.float16)
    ks, vs = 0.125, 4.0
    lut = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    kf = (lut[kc] * ks).astype(np.float16)
    vf = (lut[vc] * vs).astype(np.float16)
    assert np.array_equal(vf.astype(np.float64), lut[vc] * vs)   # exact in F16
    a = oracle.prefill_e4m3(q, kc, vc, tables, starts, lens, 0.4, bs, ks, vs)
    b = oracle.prefill(q, kf, vf, tables, starts, lens, 0.4, bs)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    with pytest.raises(ValueError):                   # a chunk longer than its sequence
        oracle.prefill_e4m3(q[:4], kc, vc, tables[:2], [0, 1, 4], [8, 2], 0.4, bs, ks, vs)
