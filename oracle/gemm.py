"""W8A8 linear layer over the quantized operands (CPU oracle).

FP8 block-scaled (FP8-RL, abstract, item (i): FP8 W8A8 linear layers with
blockwise quantization).  With ``Aq [M, K]`` e4m3 codes and ``sa [M, K/128]``
per-token-group scales, ``Wq [N, K]`` codes and ``sw [N/128, K/128]``
per-block scales (the weight is stored ``[N, K]``, K contiguous):

    C64[m, n] = sum_kb  sa[m, kb] * sw[n // 128, kb] * P(m, n, kb)
    P(m, n, kb) = sum_{k in block kb} D(Aq[m, k]) * D(Wq[n, k])

in float64, and the output is ``C64`` rounded once to bf16 (nearest, ties
to even).  Every decoded e4m3 value is a multiple of 2^-9 below 2^9, so each
product is a multiple of 2^-18 of magnitude <= 448^2 and a 128-term sum
needs at most 43 significant bits: ``P`` is exact in float64 whatever order
the matmul adds in.  ``sa * sw`` (two float32) is exact in float64 too, so
the only roundings are the final ``* P``, the sum over K-blocks and the
bf16 rounding.

INT8 per-channel (FlashRL article, INT8 rollout):

    acc[m, n] = sum_k Aq[m, k] * Wq[n, k]          (exact integer)
    C64[m, n] = acc[m, n] * (sa[m] * sw[n])

|acc| <= 127^2 K < 2^53 for K <= 2^53 / 127^2, so a float64 matmul of the
int8 values returns ``acc`` exactly, whatever its summation order.
"""

from __future__ import annotations

import numpy as np

from . import e4m3

BLOCK = 128
_DECODE = e4m3.decode(np.arange(256))


def _rows(x: np.ndarray, rows) -> np.ndarray:
    return x if rows is None else x[np.asarray(rows)]


def w8a8_block_gemm(aq, sa, wq, sw, rows=None) -> np.ndarray:
    """C64 [M or len(rows), N] (float64) of the FP8 block-scaled GEMM."""
    aq = _rows(np.asarray(aq, dtype=np.uint8), rows)
    sa = _rows(np.asarray(sa, dtype=np.float32), rows)
    wq = np.asarray(wq, dtype=np.uint8)
    sw = np.asarray(sw, dtype=np.float32)
    M, K = aq.shape
    N, K2 = wq.shape
    if K != K2 or K % BLOCK:
        raise ValueError("w8a8_block_gemm: K mismatch or K % 128 != 0")
    if np.any((aq & 0x7F) == 0x7F) or np.any((wq & 0x7F) == 0x7F):
        raise ValueError("w8a8_block_gemm: NaN code in an operand")
    kb_count = K // BLOCK
    nblk = np.arange(N) // BLOCK
    Ad = _DECODE[aq]
    C = np.zeros((M, N), dtype=np.float64)
    for kb in range(kb_count):
        ks = slice(kb * BLOCK, (kb + 1) * BLOCK)
        Wd = _DECODE[wq[:, ks]]
        P = Ad[:, ks] @ Wd.T                                   # exact
        scale = sa[:, kb].astype(np.float64)[:, None] * \
            sw[nblk, kb].astype(np.float64)[None, :]           # exact
        C += scale * P
    return C


def int8_channel_gemm(aq, sa, wq, sw, rows=None) -> np.ndarray:
    """C64 [M or len(rows), N] (float64) of the INT8 per-channel GEMM."""
    aq = _rows(np.asarray(aq, dtype=np.int8), rows)
    sa = _rows(np.asarray(sa, dtype=np.float32), rows)
    wq = np.asarray(wq, dtype=np.int8)
    sw = np.asarray(sw, dtype=np.float32)
    K = aq.shape[1]
    if wq.shape[1] != K:
        raise ValueError("int8_channel_gemm: K mismatch")
    if 127 * 127 * K >= 2 ** 53:
        raise ValueError("int8_channel_gemm: K too large for exact fp64 sums")
    acc = aq.astype(np.float64) @ wq.astype(np.float64).T      # exact
    scale = sa.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    return acc * scale


def int8_accumulator(aq, wq) -> np.ndarray:
    """The exact integer accumulator sum_k Aq[m,k] Wq[n,k] (int64)."""
    acc = np.asarray(aq, np.int8).astype(np.float64) @ \
        np.asarray(wq, np.int8).astype(np.float64).T
    return acc.astype(np.int64)


def round_bf16(c64) -> np.ndarray:
    """Round float64 values once to bf16 (nearest, ties to even); returns
    the bf16 bit patterns (uint16).  Finite results only."""
    c = np.asarray(c64, dtype=np.float64)
    if not np.all(np.isfinite(c)):
        raise ValueError("round_bf16: non-finite value")
    # bf16 keeps 8 significant bits; its quantum at |c| in [2^e, 2^(e+1)) is
    # 2^(e-7), never below the subnormal quantum 2^-133.
    _, ex = np.frexp(c)                      # |c| = f * 2^ex, f in [0.5, 1)
    q_exp = np.maximum(ex.astype(np.int64) - 8, -133)
    quantum = np.ldexp(1.0, q_exp)
    r = np.rint(c / quantum) * quantum       # exact scaling, RNE
    if np.any(np.abs(r) > 3.3895313892515355e38):
        raise ValueError("round_bf16: overflow")
    b = r.astype(np.float32).view(np.uint32)  # r is a bf16 value: exact
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def rel_frobenius(c_bits, ref_bits) -> float:
    """||C - Cref||_F / ||Cref||_F over bf16 bit arrays."""
    c = bf16_bits_to_f64(c_bits)
    r = bf16_bits_to_f64(ref_bits)
    den = np.linalg.norm(r)
    num = np.linalg.norm(c - r)
    return float(num / den) if den > 0 else float(num)


def w8a8_block_gemm_grouped(aq, sa, wq, sw, offsets) -> np.ndarray:
    """Mixture-of-experts form of the FP8 linear layer (FP8-RL, abstract:
    the FP8 stack covers dense and MoE models).  The rows of ``Aq [M, K]``
    (and ``sa [M, K/128]``) are grouped by expert: rows
    ``offsets[e] .. offsets[e+1] - 1`` go to expert ``e``, whose weight is
    ``Wq[e] [N, K]`` with scales ``sw[e] [N/128, K/128]``.  Each group is the
    dense layer above with its own expert's weight; bf16 bits [M, N].  Rows
    outside every group (before offsets[0] or from offsets[E] on) are not
    written (zero here)."""
    offs = np.asarray(offsets, dtype=np.int64)
    E = len(offs) - 1
    M = np.asarray(aq).shape[0]
    N = np.asarray(wq).shape[1]
    out = np.zeros((M, N), dtype=np.uint16)
    for e in range(E):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        if r1 > r0:
            out[r0:r1] = round_bf16(w8a8_block_gemm(aq[r0:r1], sa[r0:r1], wq[e], sw[e]))
    return out
