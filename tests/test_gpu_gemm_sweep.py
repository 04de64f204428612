"""A seeded sweep of GEMM shapes across the dispatcher's boundaries, FP8
and INT8, against the CPU oracle through the C ABI.

The fixed shape lists elsewhere pin the layers of the workloads; this
sweep draws 24 shapes (seed 2024) so that every row-count class the
dispatcher tells apart is hit -- 1-8, 9-16, 17-32, 33-64 rows (the
persistent decode kernel at one, two and four m-tiles), 65-128 (row
pairs), 129-300 (the many-token kernel) -- with ragged N and K from 1 to 40
K blocks.  Each shape runs with the caller workspace (split over K where
the plan splits) and without it (one-pass kernels); FP8 also runs the
no-allocation call, which must equal the workspace call bit for bit.
Every output sits in a guard band that must stay untouched.  The bar is
the one test_gpu_gemm.py uses: relative Frobenius error at most 1e-3
against the fp64 oracle rounded once to bf16, and every element within one
bf16 rounding plus 1e-3 of the output's rms.
"""

import numpy as np
import pytest
import torch

from oracle import gemm, quant
from precision_rl_rollout_amd import binding, workloads
from tests.gpu_util import Guarded, announce, bits_to_dev, host

pytestmark = pytest.mark.gpu

TOL = 1e-3
_CLASSES = [(1, 8), (9, 16), (17, 32), (33, 64), (65, 128), (129, 300)]


def _shapes():
    rng = np.random.default_rng(2024)
    out = []
    for i in range(24):
        lo, hi = _CLASSES[i % len(_CLASSES)]
        M = int(rng.integers(lo, hi + 1))
        N = int(rng.integers(1, 3001))
        K = 128 * int(rng.integers(1, 41))
        out.append((M, N, K))
    return out


SHAPES = _shapes()


def _check(c_gpu, c64, label):
    cref = gemm.round_bf16(c64)
    err = gemm.rel_frobenius(c_gpu, cref)
    assert err <= TOL, f"{label}: relative Frobenius error {err:.3e} > {TOL}"
    g = gemm.bf16_bits_to_f64(c_gpu)
    rms = np.sqrt(np.mean(c64 * c64)) if c64.size else 0.0
    bad = np.abs(g - c64) > 2.0 ** -8 * np.abs(c64) + 1e-3 * rms
    assert not bad.any(), f"{label}: {int(bad.sum())} elements off, first at {np.argwhere(bad)[0]}"


def _run(fn, args, M, N, workspace):
    c = Guarded((M, N), torch.bfloat16)
    if workspace == "scratch":
        binding.w8a8_block_gemm_scratch(*args, out=c.t)
    else:
        fn(*args, out=c.t, workspace=workspace)
    out = host(c.t)
    assert c.intact(), "write outside C"
    return out


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fp8_sweep(M, N, K):
    announce(f"fp8 gemm sweep M{M} N{N} K{K}")
    p = workloads.gemm_problem(M, N, K, True, seed=M + N + K)
    aq, sa = binding.fp8_act_token_quant(bits_to_dev(p["A"]))
    wq, sw = binding.fp8_weight_block_quant(bits_to_dev(p["Wt"]))
    c64 = gemm.w8a8_block_gemm(*quant.fp8_act_token_quant(p["A"]),
                               *quant.fp8_weight_block_quant(p["Wt"]))
    args = (aq, sa, wq, sw)
    with_ws = _run(binding.w8a8_block_gemm, args, M, N, "auto")
    _check(with_ws, c64, f"fp8 M{M} N{N} K{K} workspace")
    _check(_run(binding.w8a8_block_gemm, args, M, N, None), c64, f"fp8 M{M} N{N} K{K} one-pass")
    if M <= 64:   # the no-allocation call splits exactly as the workspace call
        np.testing.assert_array_equal(_run(None, args, M, N, "scratch"), with_ws)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_int8_sweep(M, N, K):
    announce(f"int8 gemm sweep M{M} N{N} K{K}")
    p = workloads.gemm_problem(M, N, K, True, seed=M + N + K + 1)
    aq, sa = binding.int8_act_token_quant(bits_to_dev(p["A"]))
    wq, sw = binding.int8_weight_channel_quant(bits_to_dev(p["Wt"]))
    c64 = gemm.int8_channel_gemm(*quant.int8_act_token_quant(p["A"]),
                                 *quant.int8_weight_channel_quant(p["Wt"]))
    args = (aq, sa, wq, sw)
    _check(_run(binding.w8a8_int8_channel_gemm, args, M, N, "auto"), c64,
           f"int8 M{M} N{N} K{K} workspace")
    _check(_run(binding.w8a8_int8_channel_gemm, args, M, N, None), c64,
           f"int8 M{M} N{N} K{K} one-pass")
