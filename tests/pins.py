"""Independent references used to pin the oracle.

Nothing here shares code with ``oracle/``; each routine reaches the same
result by a different route (exact rational arithmetic, exhaustive search
over the code book, library casts), so that a slip in the oracle shows up as
a disagreement.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch


# ---------------------------------------------------------------- e4m3 book
def e4m3_book() -> list[tuple[int, Fraction]]:
    """The 127 non-negative finite e4m3 codes and their exact values,
    enumerated from the field layout: value = 2^(E-7) * (1 + M/8) for
    E >= 1, 2^-6 * (M/8) for E = 0; code 0x7F is NaN."""
    out = []
    for code in range(0x7F):
        E, M = code >> 3, code & 7
        if E == 0:
            val = Fraction(M, 8) * Fraction(1, 64)
        else:
            val = Fraction(8 + M, 8) * (Fraction(2) ** (E - 7))
        out.append((code, val))
    return out


_BOOK = e4m3_book()
_BOOK_VALS = np.array([float(v) for _, v in _BOOK])


def e4m3_nearest(vals: np.ndarray) -> np.ndarray:
    """Brute force: nearest finite e4m3 value (saturating: anything above
    448 goes to 448), ties to the code with an even mantissa; sign kept."""
    v = np.asarray(vals, dtype=np.float64).ravel()
    if v.size > 65536:
        return np.concatenate([e4m3_nearest(v[i:i + 65536])
                               for i in range(0, v.size, 65536)])
    # beyond 448 every finite code is farther than 448 itself; clamping
    # first keeps the float64 distances from absorbing the small values
    a = np.minimum(np.abs(v), 448.0)
    d = np.abs(a[:, None] - _BOOK_VALS[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.arange(0x7F)
    # among equally near codes (at most two), pick the even one
    even = cand & ((codes[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    sign = np.signbit(v).astype(np.int64) << 7
    return (codes[pick] | sign).astype(np.uint8)


def e4m3_float_route(vals: np.ndarray) -> np.ndarray:
    """Float route: Q = rint(a / 2^(t-3)) with t = max(floor(log2 a), -6),
    in float64 with exact power-of-two scaling; saturate at 448."""
    v = np.asarray(vals, dtype=np.float32).astype(np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        t = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
    # log2 of an exact power of two is exact, but guard the floor anyway
    t = np.where(np.exp2(t) > a, t - 1, t)
    t = np.where(np.exp2(t + 1) <= a, t + 1, t)
    t = np.maximum(t, -6)
    Q = np.rint(a / np.exp2(t - 3))
    val = np.minimum(Q * np.exp2(t - 3), 448.0)
    val = np.where(a == 0, 0.0, val)
    return e4m3_nearest(np.where(np.signbit(v), -val, val))


def e4m3_torch_cast(vals: np.ndarray) -> np.ndarray:
    """Library route: torch.float8_e4m3fn cast of clamp(v, -448, 448)."""
    t = torch.from_numpy(np.asarray(vals, dtype=np.float32).copy())
    t = torch.clamp(t, -448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ------------------------------------------------------ exact binary32 round
def fl32(x: Fraction) -> np.float32:
    """Round an exact rational to binary32, nearest with ties to even,
    including subnormals, by integer arithmetic."""
    if x == 0:
        return np.float32(0.0)
    neg = x < 0
    a = -x if neg else x
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    q_exp = max(e - 23, -149)            # quantum of the target binade
    scaled = a / (Fraction(2) ** q_exp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = np.float32(float(n * (Fraction(2) ** q_exp)))   # exact: n < 2^24
    assert Fraction(float(r)) == n * (Fraction(2) ** q_exp), "not representable"
    return np.float32(-r) if neg else r


def bf16_of_fraction(x: Fraction) -> int:
    """bf16 bits of an exact rational rounded once (nearest, ties even)."""
    if x == 0:
        return 0
    neg = x < 0
    a = -x if neg else x
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    q_exp = max(e - 7, -133)
    scaled = a / (Fraction(2) ** q_exp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    f = np.float32(float(n * (Fraction(2) ** q_exp)))
    bits = int(np.array([f], dtype=np.float32).view(np.uint32)[0]) >> 16
    return bits | (0x8000 if neg else 0)


def f32_of_bf16(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)
