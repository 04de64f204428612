"""GPU parity of the W8A8 GEMMs at the limits the boundary accepts, through
the C ABI, against the CPU oracle.

* INT8 at the largest K whose products cannot overflow the int32
  accumulator (the boundary refuses K above 133,143; the largest multiple of
  128 below is 133,120): with every code at magnitude 127 each dot product
  reaches 127^2 x 133,120 = 2,147,082,880, 400,767 below 2^31, on each path
  that takes such a K -- the skinny kernel (no workspace), split-K with int32
  partial sums added exactly by the second kernel (workspace), the
  many-token kernel (more than 128 rows, and 100 rows, whose K is beyond the
  registers of the 65-128-row decode kernel).  All-positive codes make every
  product add up to the bound; a seeded sign pattern checks that the
  cancellations are exact too.
* FP8 at the longest K of the skinny kernel's LDS-staged activation scales
  (81,920 at 64 rows), and beyond it, where 64 rows run on the many-token
  kernel's mostly empty 256-row tiles, or split-K with a workspace; and 100
  rows at the same K, on the many-token kernel.
"""

import numpy as np
import pytest
import torch

from oracle import gemm, quant
from precision_rl_rollout_amd import binding, workloads
from tests.gpu_util import Guarded, announce, bits_to_dev, f32_to_dev, host, i8_to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3
INT8_K_MAX = 133120


def _check(c_gpu, c64, label):
    cref = gemm.round_bf16(c64)
    err = gemm.rel_frobenius(c_gpu, cref)
    print(f"  {label}: rel_fro vs bf16(oracle) = {err:.3e}", flush=True)
    assert err <= TOL, f"{label}: relative Frobenius error {err:.3e} > {TOL}"
    g = gemm.bf16_bits_to_f64(c_gpu)
    rms = np.sqrt(np.mean(c64 * c64))
    bad = np.abs(g - c64) > 2.0 ** -8 * np.abs(c64) + 1e-3 * rms
    assert not bad.any(), f"{label}: {int(bad.sum())} elements off, first at {np.argwhere(bad)[0]}"


def _int8_codes(rows, K, signs, rng):
    if signs == "positive":
        return np.full((rows, K), 127, dtype=np.int8)
    return np.where(rng.integers(0, 2, size=(rows, K)) == 1, -127, 127).astype(np.int8)


@pytest.mark.parametrize("M,N", [(1, 200), (40, 300), (100, 260), (200, 260)])
@pytest.mark.parametrize("signs", ["positive", "mixed"])
def test_int8_gemm_at_the_accumulator_bound(M, N, signs):
    rng = np.random.default_rng([M, N, 0 if signs == "positive" else 1])
    K = INT8_K_MAX
    aq = _int8_codes(M, K, signs, rng)
    wq = _int8_codes(N, K, signs, rng)
    # Scales that keep the outputs normal bf16 values near 1 in magnitude.
    sa = (2.0 ** -16 * (1.0 + rng.random(M))).astype(np.float32)
    sw = (2.0 ** -15 * (1.0 + rng.random(N))).astype(np.float32)
    c64 = gemm.int8_channel_gemm(aq, sa, wq, sw)
    acc = gemm.int8_accumulator(aq, wq)
    assert int(np.abs(acc).max()) <= 127 * 127 * K < 2 ** 31
    if signs == "positive":
        assert np.all(acc == 127 * 127 * K)
    a_d, w_d, sa_d, sw_d = i8_to_dev(aq), i8_to_dev(wq), f32_to_dev(sa), f32_to_dev(sw)
    for ws in ([None, "auto"] if M <= 64 else [None]):
        label = f"int8 M{M} N{N} K{K} {signs} workspace={ws}"
        announce(f"w8a8_int8_channel_gemm {label}")
        c = Guarded((M, N), torch.bfloat16)
        binding.w8a8_int8_channel_gemm(a_d, sa_d, w_d, sw_d, out=c.t, workspace=ws)
        out = host(c.t)
        assert c.intact(), "write outside C"
        _check(out, c64, label)


@pytest.mark.parametrize("M,N,K", [(64, 300, 81920), (64, 130, 90112), (7, 129, 90112),
                                   (100, 300, 90112)])
def test_fp8_gemm_long_k(M, N, K):
    p = workloads.gemm_problem(M, N, K, outliers=True, seed=5)
    aq, sa = quant.fp8_act_token_quant(p["A"])
    wq, sw = quant.fp8_weight_block_quant(p["Wt"])
    c64 = gemm.w8a8_block_gemm(aq, sa, wq, sw)
    a_dev = binding.fp8_act_token_quant(bits_to_dev(p["A"]))
    w_dev = binding.fp8_weight_block_quant(bits_to_dev(p["Wt"]))
    for ws in (None, "auto"):
        label = f"fp8 M{M} N{N} K{K} workspace={ws}"
        announce(f"w8a8_block_gemm {label}")
        c = Guarded((M, N), torch.bfloat16)
        binding.w8a8_block_gemm(*a_dev, *w_dev, out=c.t, workspace=ws)
        out = host(c.t)
        assert c.intact(), "write outside C"
        _check(out, c64, label)
