"""Pins for the oracle's FP8 block / token-group and INT8 quantizers (CPU).

* brute force with exact rational arithmetic (scale and quotient rounded
  to binary32 by integer arithmetic, code by nearest-code search);
* special blocks: all-zero, saturating, exact-e4m3 block (scale 1),
  bf16-max and bf16-subnormal amax;
* invariants: the amax element encodes to +-448, sign symmetry,
  power-of-two equivariance, shard commutation;
* the round-trip bound of half an e4m3 ulp times the scale.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, quant
from precision_rl_rollout_amd import workloads
from tests import pins


def _brute_block(xbits: np.ndarray, div: int):
    """Exact-rational reference for one block: (scale, quotients)."""
    x = pins.f32_of_bf16(xbits).ravel()
    fr = [Fraction(float(v)) for v in x]
    amax = max(abs(f) for f in fr)
    s = pins.fl32(amax / div)
    if s == 0:
        q = x.astype(np.float32)
    else:
        S = Fraction(float(s))
        q = np.array([pins.fl32(f / S) for f in fr], dtype=np.float32)
        # IEEE: x / s with s > 0 carries the sign of x, zeros included
        q = np.copysign(q, x).astype(np.float32)
    return s, q


def _rand_bits(shape, seed, sigma=0.02):
    return workloads.bf16_normal(shape, sigma, seed, "special")


# ------------------------------------------------------------ brute force
@pytest.mark.parametrize("shape", [(3, 5), (128, 128), (130, 200), (1, 129)])
def test_fp8_weight_quant_matches_brute_force(shape):
    w = _rand_bits(shape, seed=sum(shape))
    codes, scales = quant.fp8_weight_block_quant(w)
    N, K = shape
    assert scales.shape == (-(-N // 128), -(-K // 128))
    for i in range(scales.shape[0]):
        for j in range(scales.shape[1]):
            blk = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            s, q = _brute_block(blk, 448)
            assert scales[i, j] == s and np.signbit(scales[i, j]) == np.signbit(s)
            want = pins.e4m3_nearest(q).reshape(blk.shape)
            assert np.array_equal(codes[i * 128:(i + 1) * 128,
                                        j * 128:(j + 1) * 128], want)


@pytest.mark.parametrize("shape", [(2, 128), (3, 300), (16, 256)])
def test_fp8_act_quant_matches_brute_force(shape):
    a = workloads.activation(*shape, seed=7, outliers=shape[1] >= 256)
    codes, scales = quant.fp8_act_token_quant(a)
    M, K = shape
    assert scales.shape == (M, -(-K // 128))
    for m in range(M):
        for j in range(scales.shape[1]):
            grp = a[m, j * 128:(j + 1) * 128]
            s, q = _brute_block(grp, 448)
            assert scales[m, j] == s
            assert np.array_equal(codes[m, j * 128:(j + 1) * 128], pins.e4m3_nearest(q))


@pytest.mark.parametrize("shape", [(4, 37), (3, 1000)])
def test_int8_quant_matches_brute_force(shape):
    w = _rand_bits(shape, seed=3)
    for fn in (quant.int8_weight_channel_quant, quant.int8_act_token_quant):
        codes, scales = fn(w)
        assert codes.dtype == np.int8 and scales.shape == (shape[0],)
        for r in range(shape[0]):
            s, q = _brute_block(w[r], 127)
            assert scales[r] == s
            want = [max(-127, min(127, round(Fraction(float(v))))) for v in q]
            assert codes[r].tolist() == want


def test_int8_amax_maps_to_127_and_zero_row():
    w = _rand_bits((6, 512), seed=11)
    w[2] = 0
    w[3] = 0x8000          # -0.0 everywhere
    codes, scales = quant.int8_weight_channel_quant(w)
    x = quant.bf16_to_f32(w)
    for r in range(6):
        if r in (2, 3):
            assert scales[r] == 0 and np.all(codes[r] == 0)
            continue
        i = np.argmax(np.abs(x[r]))
        assert abs(int(codes[r, i])) == 127
        assert np.all(np.abs(codes[r].astype(int)) <= 127)


# ------------------------------------------------------------ special blocks
def test_all_zero_block_gives_zero_scale_and_signed_zero_codes():
    w = np.zeros((128, 256), dtype=np.uint16)
    w[5, 7] = 0x8000
    w[:, 128:] = _rand_bits((128, 128), seed=1)
    codes, scales = quant.fp8_weight_block_quant(w)
    assert scales[0, 0] == 0 and not np.signbit(scales[0, 0])
    blk = codes[:, :128]
    assert blk[5, 7] == 0x80
    blk2 = blk.copy()
    blk2[5, 7] = 0
    assert np.all(blk2 == 0)
    assert scales[0, 1] > 0


def test_saturating_block_all_pm_amax():
    rng = np.random.default_rng(5)
    sign = rng.integers(0, 2, size=(128, 128)).astype(np.uint16) << 15
    for mag in (0x3F80, 0x4234, 0x7F7F, 0x0001):    # 1.0, 45.0, bf16 max, min subnormal
        w = (sign | np.uint16(mag)).astype(np.uint16)
        codes, _ = quant.fp8_weight_block_quant(w)
        want = np.where(sign != 0, 0xFE, 0x7E).astype(np.uint8)
        assert np.array_equal(codes, want), hex(mag)


def test_exact_e4m3_block_with_amax_448_has_unit_scale():
    rng = np.random.default_rng(9)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    c = rng.choice(finite, size=(128, 128))
    c[17, 33] = 0x7E
    vals = pins.e4m3_torch_decode(c).astype(np.float32)
    bits = (vals.view(np.uint32) >> np.uint32(16)).astype(np.uint16)   # exact in bf16
    codes, scales = quant.fp8_weight_block_quant(bits)
    assert scales[0, 0] == 1.0
    assert np.array_equal(codes, c.astype(np.uint8))


def test_bf16_extreme_blocks():
    # bf16 max amax: the scale is huge but normal; bf16-subnormal amax: the
    # scale is a float32 subnormal.  Both must keep the +-448 invariant.
    for amax_bits in (0x7F7F, 0x0003, 0x0080):
        w = _rand_bits((128, 128), seed=amax_bits) & np.uint16(0x807F)
        w[0, 0] = amax_bits
        x = quant.bf16_to_f32(w)
        w = np.where(np.abs(x) > quant.bf16_to_f32(np.array([amax_bits]))[0],
                     np.uint16(amax_bits), w).astype(np.uint16)
        codes, scales = quant.fp8_weight_block_quant(w)
        s, q = _brute_block(w, 448)
        assert scales[0, 0] == s
        assert np.array_equal(codes.ravel(), pins.e4m3_nearest(q))
        assert codes[0, 0] == 0x7E


# ------------------------------------------------------------ invariants
def _blocks(codes, scales, x):
    nb, kb = scales.shape
    for i in range(nb):
        for j in range(kb):
            sl = (slice(i * 128, (i + 1) * 128), slice(j * 128, (j + 1) * 128))
            yield codes[sl], scales[i, j], x[sl]


def test_amax_element_encodes_to_448():
    w = workloads.weight(384, 512, seed=2)
    codes, scales = quant.fp8_weight_block_quant(w)
    x = quant.bf16_to_f32(w)
    for c, s, xb in _blocks(codes, scales, x):
        i = np.unravel_index(np.argmax(np.abs(xb)), xb.shape)
        assert (c[i] & 0x7F) == 0x7E
        assert np.max(c & 0x7F) == 0x7E


def test_sign_symmetry():
    w = workloads.weight(256, 384, seed=4)
    codes, scales = quant.fp8_weight_block_quant(w)
    codes_n, scales_n = quant.fp8_weight_block_quant(w ^ np.uint16(0x8000))
    assert np.array_equal(scales, scales_n)
    assert np.array_equal(codes ^ np.uint8(0x80), codes_n)


@pytest.mark.parametrize("j", [-3, 1, 5])
def test_power_of_two_equivariance(j):
    w = workloads.weight(256, 256, seed=6)
    codes, scales = quant.fp8_weight_block_quant(w)
    x2 = quant.bf16_to_f32(w) * np.float32(2.0 ** j)          # exact
    w2 = (x2.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    codes2, scales2 = quant.fp8_weight_block_quant(w2)
    assert np.array_equal(codes, codes2)
    assert np.array_equal(scales * np.float32(2.0 ** j), scales2)


def test_shard_commutation():
    w = workloads.weight(512, 640, seed=8)
    codes, scales = quant.fp8_weight_block_quant(w)
    sub = w[128:384, 256:640]
    c2, s2 = quant.fp8_weight_block_quant(sub)
    assert np.array_equal(c2, codes[128:384, 256:640])
    assert np.array_equal(s2, scales[1:3, 2:5])
    one = quant.fp8_weight_blocks(w, [(3, 4), (0, 1)])
    assert np.array_equal(one[0][0], codes[384:512, 512:640]) and one[0][1] == scales[3, 4]
    assert np.array_equal(one[1][0], codes[0:128, 128:256]) and one[1][1] == scales[0, 1]


def _half_ulp(v):
    a = np.abs(v.astype(np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.exp2(np.maximum(e, -6) - 3) / 2


def test_round_trip_bound():
    w = workloads.weight(256, 512, seed=12)
    a = workloads.activation(32, 512, seed=12)
    for bits, fn in ((w, quant.fp8_weight_block_quant), (a, quant.fp8_act_token_quant)):
        codes, scales = fn(bits)
        x = quant.bf16_to_f32(bits)
        rows, cols = x.shape
        rb = 128 if fn is quant.fp8_weight_block_quant else 1
        s_full = np.repeat(np.repeat(scales, rb, axis=0), 128, axis=1)[:rows, :cols]
        v = (x / s_full).astype(np.float32)
        dq = e4m3.decode(codes)
        # exact form: |fl32(x/s) - D(q)| <= half an e4m3 ulp of the quotient
        assert np.all(np.abs(v.astype(np.float64) - dq) <= _half_ulp(v))
        # against raw x: the scale times half an ulp, plus the fp32 quotient's rounding
        s64 = s_full.astype(np.float64)
        x64 = x.astype(np.float64)
        assert np.all(np.abs(x64 - dq * s64) <= s64 * _half_ulp(v) + 2.0 ** -24 * np.abs(x64) * 1.0001)


def test_non_finite_input_is_rejected():
    w = np.zeros((4, 4), dtype=np.uint16)
    w[1, 1] = 0x7F80          # +inf
    with pytest.raises(ValueError):
        quant.fp8_weight_block_quant(w)
    with pytest.raises(ValueError):
        quant.int8_act_token_quant(w)
