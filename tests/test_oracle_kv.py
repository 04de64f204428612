"""Pins for the oracle's FP8 KV-cache scale recalibration and quantize-on-write
(CPU).

* brute force with exact rational arithmetic: amax and scale rounded to
  binary32 by integer arithmetic, quotients likewise, codes by nearest-code
  search;
* special tensors: all zero (scale 0, signed-zero codes), values beyond the
  calibration range (saturation to +-448), an exact-e4m3 tensor;
* scatter semantics against a hand-built expectation: padding (negative)
  and out-of-range slots skipped, untouched rows kept, duplicate slots
  refused;
* the round-trip bound of half an e4m3 ulp times the scale.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, kv
from precision_rl_rollout_amd import workloads
from tests import pins


def _bits(shape, seed, sigma=1.0):
    return workloads.bf16_normal(shape, sigma, seed, "special")


def _brute_scale_and_quotients(xbits):
    x = pins.f32_of_bf16(xbits).ravel()
    fr = [Fraction(float(v)) for v in x]
    amax = max((abs(f) for f in fr), default=Fraction(0))
    s = pins.fl32(amax / 448)
    if s == 0:
        return s, x.astype(np.float32)
    S = Fraction(float(s))
    q = np.array([pins.fl32(f / S) for f in fr], dtype=np.float32)
    return s, np.copysign(q, x).astype(np.float32)


@pytest.mark.parametrize("shape", [(1, 8), (3, 40), (7, 128), (5, 1000)])
def test_scale_and_codes_match_brute_force(shape):
    xb = _bits(shape, seed=sum(shape))
    s, q = _brute_scale_and_quotients(xb)
    assert kv.kv_scale(xb) == s
    assert np.array_equal(kv.kv_encode_rows(xb, s).ravel(), pins.e4m3_nearest(q))


def test_all_zero_tensor():
    xb = np.zeros((4, 16), dtype=np.uint16)
    xb[1, 3] = 0x8000                               # -0.0
    s = kv.kv_scale(xb)
    assert s == 0 and not np.signbit(s)
    codes = kv.kv_encode_rows(xb, s)
    want = np.zeros((4, 16), dtype=np.uint8)
    want[1, 3] = 0x80
    assert np.array_equal(codes, want)


def test_zero_scale_writes_signed_zeros_of_nonzero_rows():
    xb = _bits((3, 10), seed=9)
    codes = kv.kv_encode_rows(xb, np.float32(0.0))
    x = pins.f32_of_bf16(xb)
    assert np.array_equal(codes, np.where(np.signbit(x), 0x80, 0x00).astype(np.uint8))


def test_values_beyond_calibration_saturate():
    cal = _bits((16, 64), seed=11)
    s = kv.kv_scale(cal)
    x = pins.f32_of_bf16(cal)
    big = np.array([[4.0, -4.0, 1.5, -1.5]], dtype=np.float32) * np.max(np.abs(x))
    bits = (big.view(np.uint32) >> 16).astype(np.uint16)   # exact: powers of two times bf16
    codes = kv.kv_encode_rows(bits, s)
    assert list(codes[0]) == [0x7E, 0xFE, 0x7E, 0xFE]


def test_quotients_beyond_binary32_saturate():
    # A stale scale far below the new values: fl32(x / s) overflows to
    # +-inf, which is a value above the calibrated range and saturates.
    s = np.float32(np.float32(2.0 ** -120) / np.float32(448))
    bits = np.array([[0x3F80, 0xBF80, 0x7F7F, 0xFF7F, 0x0000, 0x8000]], dtype=np.uint16)
    codes = kv.kv_encode_rows(bits, s)
    assert list(codes[0]) == [0x7E, 0xFE, 0x7E, 0xFE, 0x00, 0x80]
    # brute force: every code is the saturating code of the exact rational
    # quotient, which here is far above 448 for the nonzero values
    x = pins.f32_of_bf16(bits).astype(np.float64)
    assert np.all(np.abs(x[0, :4]) / float(s) > 3.4e38)


def test_exact_e4m3_values_round_trip():
    # amax 448 gives s = 1: every e4m3 value is its own quotient
    vals = np.array([float(v) for _, v in pins.e4m3_book()], dtype=np.float32)
    vals = np.concatenate([vals, -vals])
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)[None, :]
    assert kv.kv_scale(bits) == 1.0
    codes = kv.kv_encode_rows(bits, np.float32(1.0))
    assert np.array_equal(e4m3.decode(codes).astype(np.float32), pins.f32_of_bf16(bits))


def test_round_trip_bound():
    xb = _bits((64, 256), seed=5)
    s = kv.kv_scale(xb)
    codes = kv.kv_encode_rows(xb, s)
    x = pins.f32_of_bf16(xb).astype(np.float64)
    back = e4m3.decode(codes) * float(s)
    # half an e4m3 ulp of the quotient (2^-10 below the normal range), times s,
    # plus the quotient's own binary32 rounding
    q = np.abs(x) / float(s)
    e = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    half_ulp = 2.0 ** (e - 4)
    assert np.all(np.abs(back - x) <= (half_ulp * (1 + 2.0 ** -22) + 2.0 ** -24 * q) * float(s))


def test_cache_write_scatter_semantics():
    xb = _bits((4, 3), seed=2)
    s = kv.kv_scale(xb)
    cache = np.full((5, 3), 0x5A, dtype=np.uint8)
    slots = np.array([3, -1, 0, 7])                 # a padding token, one past the cache
    got = kv.kv_cache_write(cache, xb, slots, s)
    _, q = _brute_scale_and_quotients(xb)
    codes = pins.e4m3_nearest(q).reshape(4, 3)
    want = cache.copy()
    want[3] = codes[0]
    want[0] = codes[2]
    assert np.array_equal(got, want)
    assert np.array_equal(cache, np.full((5, 3), 0x5A, dtype=np.uint8))   # input untouched


def test_cache_write_refuses_duplicate_slots():
    xb = _bits((2, 4), seed=3)
    with pytest.raises(ValueError):
        kv.kv_cache_write(np.zeros((4, 4), np.uint8), xb, np.array([1, 1]), kv.kv_scale(xb))
