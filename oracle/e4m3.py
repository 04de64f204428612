"""OCP FP8 E4M3 ("e4m3fn") codec, written from the format's definition.

Format: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
field 0 holds subnormals ``m * 2^-9``; fields 1..15 hold normals
``(8 + m) * 2^(e - 10)``; ``S.1111.111`` is NaN and there is no infinity, so
the largest finite magnitude is ``S.1111.110`` = 448.  This is the format
the blockwise FP8 rollout of "FP8-RL: A Practical and Stable Low-Precision
Stack for LLM Reinforcement Learning" (abstract, item (i)) is read to use,
with scale constant 448.

Encoding is saturating round-to-nearest, ties to even: magnitudes at or
above 448 give 448 (never NaN), the sign is kept (``-0`` -> 0x80).  It is
built from the float32 fields with integer shifts and explicit round and
sticky bits, not with any float cast.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
CODE_MAX = 0x7E          # +448
NAN_CODES = (0x7F, 0xFF)


def encode(v) -> np.ndarray:
    """Saturating RNE e4m3 code (uint8) of float32 values ``v``.

    Steps, per element:
      1. sign = sign bit of v, a = |v|.
      2. a >= 448 -> code 0x7E (saturate).
      3. a below the float32 normal range (fields exponent 0, so
         a < 2^-126 < 2^-10) -> code 0 (rounds to zero).
      4. otherwise a = S * 2^(e - 23) with S = 2^23 | mantissa.  The target
         exponent is t = max(e, -6) (-6 is e4m3's smallest normal exponent)
         and the target quantum is 2^(t - 3), i.e. a shift of
         sh = 20 + t - e bits out of S.  Q = S >> sh, rounded to nearest
         with ties to even from the dropped bits.
      5. Q < 8 (only when t = -6): subnormal, code = Q.
         Q == 16: the mantissa carried into the next binade, Q = 8, t += 1.
         code = ((t + 7) << 3) | (Q - 8).
      6. OR in sign << 7.
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    bits = v.view(np.uint32).astype(np.int64)
    sign = (bits >> 31) & 1
    abits = bits & 0x7FFFFFFF
    if np.any(abits >= 0x7F800000):
        raise ValueError("e4m3.encode: non-finite input")
    efield = abits >> 23
    mant = abits & 0x7FFFFF

    e = efield - 127
    S = (1 << 23) | mant
    t = np.maximum(e, -6)
    sh = 20 + t - e                       # >= 20 for every normal input
    big = sh >= 25                        # S < 2^24 <= 2^(sh-1): rounds to 0
    shc = np.minimum(sh, 24)
    Q = S >> shc
    rem = S & ((1 << shc) - 1)
    half = 1 << (shc - 1)
    round_up = (rem > half) | ((rem == half) & ((Q & 1) == 1))
    Q = Q + round_up.astype(np.int64)
    Q = np.where(big, 0, Q)

    carry = Q == 16
    Q = np.where(carry, 8, Q)
    t = np.where(carry, t + 1, t)
    normal_code = ((t + 7) << 3) | (Q - 8)
    code = np.where(Q < 8, Q, normal_code)

    code = np.where(efield == 0, 0, code)          # float32 zero / subnormal
    code = np.where(abits >= np.float32(E4M3_MAX).view(np.uint32).astype(np.int64),
                    CODE_MAX, code)
    code = code | (sign << 7)
    return code.astype(np.uint8)


def decode(c) -> np.ndarray:
    """Exact value (float64) of e4m3 codes; NaN for 0x7F / 0xFF."""
    c = np.asarray(c).astype(np.int64)
    ef = (c >> 3) & 15
    m = c & 7
    mag = np.where(ef == 0, m * 2.0 ** -9, (8 + m) * np.exp2(ef - 10.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where((c >> 7) & 1 == 1, -mag, mag)


def decode_units(c) -> np.ndarray:
    """Exact value of e4m3 codes as an integer multiple of 2^-9 (int64).

    Every finite e4m3 value is such a multiple: subnormal m * 2^-9, normal
    (8 + m) * 2^(ef - 1) * 2^-9.
    """
    c = np.asarray(c).astype(np.int64)
    if np.any((c & 0x7F) == 0x7F):
        raise ValueError("e4m3.decode_units: NaN code")
    ef = (c >> 3) & 15
    m = c & 7
    mag = np.where(ef == 0, m, (8 + m) << np.maximum(ef - 1, 0))
    return np.where((c >> 7) & 1 == 1, -mag, mag)
