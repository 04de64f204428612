"""Pins for the oracle's W8A8 GEMMs and its bf16 rounding (CPU only).

* exact rational arithmetic on small non-square problems: every e4m3 value
  is an integer multiple of 2^-9 (taken from the field-layout code book,
  not from the oracle's decoder) and every fp32 scale is a dyadic rational,
  so the exact C is computable with Python integers;
* special case scales = 1: the textbook fp64 matmul of torch-decoded codes;
* the bf16 rounding against torch's float32 -> bf16 cast and against an
  exact-rational rounding;
* agreement with the unquantized bf16 GEMM within the quantization bound;
* planted mistakes (a wrong scale index, a dropped K-block, a transposed
  operand) are caught by the exact check.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import gemm, quant
from precision_rl_rollout_amd import workloads
from tests import pins

_UNITS = {c: int(v * 512) for c, v in pins.e4m3_book()}


def _units(codes):
    u = np.vectorize(lambda c: _UNITS[c & 0x7F] * (-1 if c & 0x80 else 1))(codes)
    return u.astype(np.int64)


def _exact_fp8(aq, sa, wq, sw):
    """Exact C as Fractions (object array), and sum_kb |term| (float)."""
    M, K = aq.shape
    N = wq.shape[0]
    ua, uw = _units(aq), _units(wq)
    out = np.empty((M, N), dtype=object)
    mag = np.zeros((M, N))
    P = [ua[:, kb * 128:(kb + 1) * 128] @ uw[:, kb * 128:(kb + 1) * 128].T
         for kb in range(K // 128)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for kb in range(K // 128):
                term = Fraction(float(sa[m, kb])) * Fraction(float(sw[n // 128, kb])) \
                    * int(P[kb][m, n])
                acc += term
                mag[m, n] += float(abs(term))
            out[m, n] = acc / (1 << 18)
            mag[m, n] /= 1 << 18
    return out, mag


def _problem(M, N, K, seed, outliers=False):
    p = workloads.gemm_problem(M, N, K, outliers, seed)
    aq, sa = quant.fp8_act_token_quant(p["A"])
    wq, sw = quant.fp8_weight_block_quant(p["Wt"])
    return p, aq, sa, wq, sw


def _exact_check(fn, aq, sa, wq, sw, exact_mag):
    """fn's C64 within 2^-50 * sum_kb |term| of the exact C, everywhere."""
    exact, mag = exact_mag
    c64 = fn(aq, sa, wq, sw)
    if c64.shape != exact.shape:
        return False
    err = np.abs(c64 - np.vectorize(float)(exact))
    return bool(np.all(err <= 2.0 ** -50 * mag))


@pytest.mark.parametrize("M,N,K", [(16, 384, 256), (3, 130, 384)])
def test_fp8_gemm_matches_exact_rational(M, N, K):
    p, aq, sa, wq, sw = _problem(M, N, K, seed=M + N)
    exact = _exact_fp8(aq, sa, wq, sw)
    assert _exact_check(gemm.w8a8_block_gemm, aq, sa, wq, sw, exact)
    ref = gemm.round_bf16(gemm.w8a8_block_gemm(aq, sa, wq, sw))
    want = np.vectorize(pins.bf16_of_fraction)(exact[0]).astype(np.uint16)
    assert np.array_equal(ref, want)


def test_fp8_gemm_row_subset():
    p, aq, sa, wq, sw = _problem(16, 256, 256, seed=1)
    full = gemm.w8a8_block_gemm(aq, sa, wq, sw)
    sub = gemm.w8a8_block_gemm(aq, sa, wq, sw, rows=[3, 0, 15])
    assert np.array_equal(sub, full[[3, 0, 15]])


# Planted mistakes: each variant below is the oracle's GEMM with one slip.
def _mut_scale_index(aq, sa, wq, sw):
    dq = pins.e4m3_torch_decode
    M, K = aq.shape
    N = wq.shape[0]
    C = np.zeros((M, N))
    for kb in range(K // 128):
        ks = slice(kb * 128, (kb + 1) * 128)
        P = dq(aq[:, ks]) @ dq(wq[:, ks]).T
        C += sa[:, kb, None].astype(float) * sw[np.arange(N) % sw.shape[0], kb][None].astype(float) * P
    return C


def _mut_drop_block(aq, sa, wq, sw):
    return gemm.w8a8_block_gemm(aq[:, :-128], sa[:, :-1], wq[:, :-128], sw[:, :-1])


def _mut_transposed_weight(aq, sa, wq, sw):
    # the [N, K] buffer read as if it were stored [K, N]
    N, K = wq.shape
    return gemm.w8a8_block_gemm(aq, sa, np.ascontiguousarray(wq.reshape(K, N).T), sw)


@pytest.mark.parametrize("mutant", [_mut_scale_index, _mut_drop_block, _mut_transposed_weight])
def test_planted_gemm_mistakes_are_caught(mutant):
    p, aq, sa, wq, sw = _problem(16, 384, 256, seed=5)
    exact = _exact_fp8(aq, sa, wq, sw)
    assert not _exact_check(mutant, aq, sa, wq, sw, exact)


def test_unit_scales_reduce_to_textbook_matmul():
    rng = np.random.default_rng(2)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    aq = rng.choice(finite, size=(8, 256))
    wq = rng.choice(finite, size=(200, 256))
    sa = np.ones((8, 2), np.float32)
    sw = np.ones((2, 2), np.float32)
    want = pins.e4m3_torch_decode(aq) @ pins.e4m3_torch_decode(wq).T
    assert np.array_equal(gemm.w8a8_block_gemm(aq, sa, wq, sw), want)


def test_agreement_with_bf16_gemm_within_quantization_bound():
    for (M, N, K, outl) in [(16, 256, 256, False), (8, 384, 1024, True)]:
        p, aq, sa, wq, sw = _problem(M, N, K, seed=K, outliers=outl)
        a = quant.bf16_to_f32(p["A"]).astype(np.float64)
        w = quant.bf16_to_f32(p["Wt"]).astype(np.float64)
        c_bf = a @ w.T
        c64 = gemm.w8a8_block_gemm(aq, sa, wq, sw)
        s_a = np.repeat(sa, 128, axis=1).astype(np.float64)
        s_w = np.repeat(np.repeat(sw, 128, axis=0), 128, axis=1)[:N].astype(np.float64)

        def eps(x, s):
            return np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * s) + 2.0 ** -24 * np.abs(x)
        ea, ew = eps(a, s_a), eps(w, s_w)
        bound = ea @ np.abs(w).T + np.abs(a) @ ew.T + ea @ ew.T
        assert np.all(np.abs(c64 - c_bf) <= bound * (1 + 1e-9))
        rel = np.linalg.norm(c64 - c_bf) / np.linalg.norm(c_bf)
        assert 1e-3 < rel < 0.08     # FP8 blockwise error is a few percent


# ------------------------------------------------------------ bf16 rounding
def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    ours = gemm.round_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_round_bf16_matches_exact_rounding_with_ties():
    rng = np.random.default_rng(1)
    base = rng.standard_normal(3000) * np.exp2(rng.integers(-30, 30, 3000))
    # exact bf16 midpoints (ties) and their fp64 neighbours
    hb = (base.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    mids = hb.astype(np.float64) + np.copysign(2.0 ** (np.floor(np.log2(np.abs(hb.astype(np.float64)))) - 8), hb)
    vals = np.concatenate([base, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                           [0.0, -0.0, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134]])
    ours = gemm.round_bf16(vals)
    want = np.array([pins.bf16_of_fraction(Fraction(float(v))) for v in vals], dtype=np.uint16)
    # the exact route drops the sign of zero; compare magnitudes there
    nz = vals != 0
    assert np.array_equal(ours[nz], want[nz])
    assert ours[-5] == 0x0000 and ours[-4] == 0x8000     # -0.0 keeps its sign


def test_rel_frobenius():
    r = gemm.round_bf16(np.array([[1.0, 2.0], [3.0, 4.0]]))
    c = gemm.round_bf16(np.array([[1.0, 2.0], [3.0, 4.5]]))
    assert gemm.rel_frobenius(r, r) == 0.0
    assert abs(gemm.rel_frobenius(c, r) - 0.5 / np.sqrt(30.0)) < 1e-12


# ------------------------------------------------------------ INT8
def test_int8_gemm_exact():
    p = workloads.gemm_problem(5, 70, 384, True, seed=4)
    aq, sa = quant.int8_act_token_quant(p["A"])
    wq, sw = quant.int8_weight_channel_quant(p["Wt"])
    acc = gemm.int8_accumulator(aq, wq)
    a_i, w_i = aq.astype(object), wq.astype(object)
    for m in range(5):
        for n in range(70):
            assert acc[m, n] == sum(int(x) * int(y) for x, y in zip(a_i[m], w_i[n]))
    c64 = gemm.int8_channel_gemm(aq, sa, wq, sw)
    for m in range(5):
        for n in range(0, 70, 7):
            ex = Fraction(int(acc[m, n])) * Fraction(float(sa[m])) * Fraction(float(sw[n]))
            assert abs(Fraction(float(c64[m, n])) - ex) <= abs(ex) * Fraction(1, 2 ** 52)
