"""Pins for the oracle's grouped (mixture-of-experts) FP8 GEMM (CPU).

* exact rational arithmetic per expert group (the dense exact check of the
  GEMM pins, applied to each group with its own expert's weight), with an
  empty expert and groups of different sizes, compared bit for bit after
  one exact rounding to bf16;
* rows outside every group are not written; one expert spanning all rows
  is the dense layer.
"""

import numpy as np

from oracle import gemm, quant
from precision_rl_rollout_amd import workloads
from tests import pins
from tests.test_oracle_gemm import _exact_fp8


def _experts(E, M, N, K, seed):
    a = workloads.activation(M, K, seed, True, "A")
    aq, sa = quant.fp8_act_token_quant(a)
    ws = [quant.fp8_weight_block_quant(workloads.weight(N, K, seed + e, "W")) for e in range(E)]
    wq = np.stack([w for w, _ in ws])
    sw = np.stack([s for _, s in ws])
    return aq, sa, wq, sw


def test_grouped_gemm_matches_exact_rational_per_expert():
    E, M, N, K = 3, 5, 130, 256
    aq, sa, wq, sw = _experts(E, M, N, K, seed=4)
    offsets = np.array([0, 2, 2, 5])           # expert 1 gets no token
    got = gemm.w8a8_block_gemm_grouped(aq, sa, wq, sw, offsets)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        exact, _ = _exact_fp8(aq[r0:r1], sa[r0:r1], wq[e], sw[e])
        want = np.vectorize(pins.bf16_of_fraction)(exact).astype(np.uint16)
        assert np.array_equal(got[r0:r1], want), e


def test_rows_outside_groups_untouched_and_single_expert_is_dense():
    E, M, N, K = 2, 6, 64, 128
    aq, sa, wq, sw = _experts(E, M, N, K, seed=7)
    got = gemm.w8a8_block_gemm_grouped(aq, sa, wq, sw, np.array([1, 3, 5]))
    assert not got[0].any() and not got[5].any()
    dense = gemm.round_bf16(gemm.w8a8_block_gemm(aq, sa, wq[0], sw[0]))
    one = gemm.w8a8_block_gemm_grouped(aq, sa, wq[:1], sw[:1], np.array([0, M]))
    assert np.array_equal(one, dense)
