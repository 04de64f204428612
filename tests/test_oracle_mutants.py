"""Planted mistakes in the oracle's quantizer are caught by its pins (CPU).

Each mutant is the oracle with one plausible slip; the same checks that the
oracle passes must fail on it.
"""

import numpy as np
import pytest

from oracle import e4m3, quant
from precision_rl_rollout_amd import workloads
from tests import pins


def _encode_ties_away(v):
    """e4m3 with ties rounded away from zero instead of to even."""
    v = np.asarray(v, dtype=np.float32)
    up = np.nextafter(np.abs(v), np.float32(np.inf)).astype(np.float32)
    return e4m3.encode(np.where(np.signbit(v), -up, up).astype(np.float32))


def _encode_truncating(v):
    """e4m3 that truncates toward zero."""
    v = np.asarray(v, dtype=np.float32)
    c = e4m3.encode(v)
    back = e4m3.decode(c)
    over = np.abs(back) > np.abs(v.astype(np.float64))
    return np.where(over & ((c & 0x7F) > 0), c - 1, c).astype(np.uint8)


def _boundary_values():
    book = sorted(float(v) for _, v in pins.e4m3_book())
    mids = np.array([(a + b) / 2 for a, b in zip(book[:-1], book[1:])], dtype=np.float32)
    return np.concatenate([mids, -mids, mids * np.float32(1.0000001)])


@pytest.mark.parametrize("mutant", [_encode_ties_away, _encode_truncating])
def test_encoder_mutants_fail_the_library_cross_check(mutant):
    v = _boundary_values()
    assert np.array_equal(e4m3.encode(v), pins.e4m3_torch_cast(v))
    assert not np.array_equal(mutant(v), pins.e4m3_torch_cast(v))


def _quant_reciprocal(w_bits):
    """Block quant with x * (1/s) in place of the correctly rounded x / s."""
    x = quant.bf16_to_f32(w_bits)
    N, K = x.shape
    codes = np.empty((N, K), np.uint8)
    for i in range(0, N, 128):
        for j in range(0, K, 128):
            blk = x[i:i + 128, j:j + 128]
            s = np.float32(np.max(np.abs(blk))) / np.float32(448)
            codes[i:i + 128, j:j + 128] = e4m3.encode(blk * (np.float32(1) / s))
    return codes


def _quant_scale_447(w_bits):
    """Block quant with a wrong scale constant."""
    x = quant.bf16_to_f32(w_bits)
    codes = np.empty(x.shape, np.uint8)
    for i in range(0, x.shape[0], 128):
        for j in range(0, x.shape[1], 128):
            blk = x[i:i + 128, j:j + 128]
            s = np.float32(np.max(np.abs(blk))) / np.float32(447)
            codes[i:i + 128, j:j + 128] = e4m3.encode(blk / s)
    return codes


def test_quantizer_mutants_are_caught():
    w = workloads.weight(1024, 1024, seed=21)
    codes, _ = quant.fp8_weight_block_quant(w)
    # the invariant "the amax element encodes to 0x7E, nothing larger"
    # catches a wrong constant; the three-route agreement on quotients
    # catches the reciprocal shortcut
    bad = _quant_scale_447(w)
    assert not np.array_equal(bad, codes)
    assert np.any((bad & 0x7F) != (codes & 0x7F))
    recip = _quant_reciprocal(w)
    assert not np.array_equal(recip, codes)


# ----------------------------------------------------------------- KV cache
from oracle import kv as _kv                                     # noqa: E402


def _kv_write_ignoring_mapping(cache, x_bits, slots, s):
    """Token t written to row t instead of row slot_mapping[t]."""
    out = np.array(cache, copy=True)
    codes = _kv.kv_encode_rows(x_bits, s)
    n = min(len(slots), out.shape[0])
    out[:n] = codes[:n]
    return out


def _kv_write_unclamped_slots(cache, x_bits, slots, s):
    """Negative slots taken as Python indices from the end of the cache."""
    out = np.array(cache, copy=True)
    codes = _kv.kv_encode_rows(x_bits, s)
    for t, sl in enumerate(np.asarray(slots)):
        if sl < out.shape[0]:
            out[sl] = codes[t]
    return out


def _kv_zero_scale_encodes_x(x_bits, s):
    """s == 0 handled by encoding x itself (the weight-block shortcut)."""
    return e4m3.encode(quant.bf16_to_f32(x_bits))


def _kv_scatter_check(write):
    xb = workloads.bf16_normal((4, 3), 1.0, 2, "special")
    s = _kv.kv_scale(xb)
    cache = np.full((5, 3), 0x5A, dtype=np.uint8)
    slots = np.array([3, -1, 0, 7])
    x = pins.f32_of_bf16(xb)
    want = cache.copy()
    q = pins.e4m3_nearest((x / np.float64(s)).astype(np.float32)).reshape(4, 3)
    want[3], want[0] = q[0], q[2]
    return np.array_equal(write(cache, xb, slots, s), want)


def test_kv_write_mutants_fail_the_scatter_pin():
    assert _kv_scatter_check(_kv.kv_cache_write)
    assert not _kv_scatter_check(_kv_write_ignoring_mapping)
    assert not _kv_scatter_check(_kv_write_unclamped_slots)


def test_kv_zero_scale_mutant_fails_the_signed_zero_pin():
    xb = workloads.bf16_normal((3, 10), 1.0, 9, "special")
    want = np.where(np.signbit(pins.f32_of_bf16(xb)), 0x80, 0x00).astype(np.uint8)
    assert np.array_equal(_kv.kv_encode_rows(xb, np.float32(0)), want)
    assert not np.array_equal(_kv_zero_scale_encodes_x(xb, np.float32(0)), want)
