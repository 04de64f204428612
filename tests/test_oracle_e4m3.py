"""Pins for the oracle's e4m3 codec (CPU only).

The encoder is checked against three other routes -- brute-force nearest
code, a float formulation, and torch's float8_e4m3fn cast -- on every finite
bf16 pattern divided by a spread of scales, on windows of float32 patterns
around every e4m3 rounding boundary, and on a stratified sweep of float32;
the decoder against the format's published code points and torch's decode.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, quant
from precision_rl_rollout_amd import workloads
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_e4m3_values.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val, *_ = line.split()
        rows.append((int(code, 16), val))
    return rows


def test_decode_matches_published_code_points():
    for code, val in _golden():
        got = e4m3.decode(np.array([code]))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            num, den = val.split("/")
            want = Fraction(int(num), int(den))
            assert Fraction(float(got)) == want, hex(code)
            if num.startswith("-"):
                assert np.signbit(got)


def test_decode_all_codes_matches_torch_and_units():
    codes = np.arange(256)
    ours = e4m3.decode(codes)
    ref = pins.e4m3_torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    finite = codes[~nan]
    units = e4m3.decode_units(finite)
    assert np.array_equal(units * 2.0 ** -9, ours[~nan])


def test_decode_matches_field_layout_book():
    for code, val in pins.e4m3_book():
        assert Fraction(float(e4m3.decode(np.array([code]))[0])) == val


def test_encode_decode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert len(codes) == 254
    vals = e4m3.decode(codes).astype(np.float32)
    assert np.array_equal(e4m3.encode(vals), codes.astype(np.uint8))


def _boundary_windows(width=1024):
    """float32 patterns in a window around every midpoint between adjacent
    non-negative e4m3 values and around 448 / 464, both signs."""
    book = sorted(float(v) for _, v in pins.e4m3_book())
    mids = [(a + b) / 2 for a, b in zip(book[:-1], book[1:])] + [448.0, 464.0, 480.0]
    out = []
    for m in mids:
        c = np.array([m], dtype=np.float32).view(np.uint32)[0].astype(np.int64)
        w = np.arange(max(c - width, 0), c + width + 1, dtype=np.int64)
        out.append(w.astype(np.uint32).view(np.float32))
    v = np.concatenate(out)
    return np.concatenate([v, -v])


def _quotients_all_bf16():
    x = quant.bf16_to_f32(workloads.special_values_bf16())
    scales = np.array([1.0, 0.75, 448.0 / 3.0, 2.0 ** -20, 1.0 / 448.0,
                       0.0137, 7.3e-5, 3.1e5], dtype=np.float32)
    with np.errstate(all="ignore"):
        q = np.concatenate([(x / s).astype(np.float32) for s in scales])
    return q[np.isfinite(q)]


def _stratified_f32(step=4099):
    """Every step-th positive float32 pattern up to 480, both signs."""
    top = np.array([480.0], dtype=np.float32).view(np.uint32)[0]
    v = np.arange(0, int(top) + 1, step, dtype=np.uint32).view(np.float32)
    return np.concatenate([v, -v])


@pytest.mark.parametrize("source", ["boundaries", "bf16_quotients", "stratified"])
def test_encode_agrees_with_three_other_routes(source):
    v = {"boundaries": _boundary_windows,
         "bf16_quotients": _quotients_all_bf16,
         "stratified": _stratified_f32}[source]()
    ours = e4m3.encode(v)
    lib = pins.e4m3_torch_cast(v)
    assert np.array_equal(ours, lib), "oracle vs torch float8_e4m3fn cast"
    sub = v if v.size <= 600_000 else v[:: v.size // 600_000 + 1]
    sub_ours = e4m3.encode(sub)
    assert np.array_equal(sub_ours, pins.e4m3_float_route(sub)), "float route"
    assert np.array_equal(sub_ours, pins.e4m3_nearest(sub)), "brute force"


def test_encode_saturates_and_never_makes_nan():
    v = np.array([448, 449, 463.9, 464, 465, 479.9, 480, 1e4, 3.39e38,
                  -448, -464, -3.39e38], dtype=np.float32)
    want = np.array([0x7E] * 9 + [0xFE] * 3, dtype=np.uint8)
    assert np.array_equal(e4m3.encode(v), want)


def test_encode_signed_zero_and_tiny():
    v = np.array([0.0, -0.0, 2.0 ** -149, -(2.0 ** -149), 2.0 ** -10,
                  -(2.0 ** -10), 2.0 ** -10 * 1.0000001, 3 * 2.0 ** -10],
                 dtype=np.float32)
    # 2^-10 is the midpoint 0 | 2^-9: ties go to the even code 0;
    # 3 * 2^-10 is the midpoint 2^-9 | 2^-8: ties go to code 2.
    want = np.array([0x00, 0x80, 0x00, 0x80, 0x00, 0x80, 0x01, 0x02], np.uint8)
    assert np.array_equal(e4m3.encode(v), want)


def test_encode_rejects_non_finite():
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.inf], dtype=np.float32))
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.nan], dtype=np.float32))
