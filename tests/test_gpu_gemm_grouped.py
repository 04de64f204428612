"""GPU parity of the grouped (mixture-of-experts) FP8 GEMM against the oracle.

Each case quantizes the inputs with the oracle, runs w8a8_block_gemm_grouped
on the same codes and scales, and compares the grouped rows with the
oracle's per-expert fp64 result rounded once to bf16 (relative Frobenius
error <= 1e-3).  The output sits in a canary-filled buffer: rows outside
every group and the margins around the output must keep the canary.  Cases:
ragged N, an empty expert, a group above 64 rows (processed in chunks), rows
before the first and after the last group, each register tiling
(max_rows_per_expert 16 / 32 / 64), K = 6144 and 8192, and a 128-expert
top-8 decode layer.
"""

import numpy as np
import pytest
import torch

from oracle import gemm, quant
from precision_rl_rollout_amd import binding, workloads
from tests.gpu_util import CANARY, Guarded, announce, host

pytestmark = pytest.mark.gpu

TOL = 1e-3
CANARY16 = CANARY * 0x0101


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _run_and_check(counts, N, K, hint, seed=0, lead=0, tail=0):
    p = workloads.moe_problem(counts, N, K, seed)
    E = len(counts)
    offsets = p["offsets"] + lead
    A = np.concatenate([np.zeros((lead, K), np.uint16), p["A"],
                        np.zeros((tail, K), np.uint16)])
    aq, sa = quant.fp8_act_token_quant(A)
    wq_sw = [quant.fp8_weight_block_quant(p["Wt"][e]) for e in range(E)]
    wq = np.stack([w for w, _ in wq_sw])
    sw = np.stack([s for _, s in wq_sw])
    ref = gemm.w8a8_block_gemm_grouped(aq, sa, wq, sw, offsets)
    M = A.shape[0]
    g = Guarded((M, N), torch.bfloat16)
    binding.w8a8_block_gemm_grouped(_dev(aq), _dev(sa), _dev(wq), _dev(sw), _dev(offsets),
                                    hint, out=g.t)
    got = host(g.t)
    assert g.intact(), "write outside the output"
    r0, r1 = int(offsets[0]), int(offsets[-1])
    assert np.all(got[:r0] == CANARY16) and np.all(got[r1:] == CANARY16), "rows outside groups"
    err = gemm.rel_frobenius(got[r0:r1], ref[r0:r1])
    assert err <= TOL, f"relative Frobenius error {err:.3e}"
    # Element by element: the two bf16 roundings (<= 2^-8 relative each) and
    # an fp32 accumulation error far below 1e-3 of the rms; a value written to
    # the wrong row or channel is off by about the rms.
    g = gemm.bf16_bits_to_f64(got[r0:r1])
    r = gemm.bf16_bits_to_f64(ref[r0:r1])
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    bad = np.abs(g - r) > 2.0 ** -7 * np.abs(r) + 1e-3 * rms
    assert not bad.any(), f"{int(bad.sum())} elements off, first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("counts,N,K,hint", [
    ([3, 0, 17, 1, 9], 300, 256, 32),
    ([16, 16, 5], 128, 1024, 16),
    ([64, 2, 40, 0, 7], 520, 512, 64),
    ([100, 3, 70], 256, 384, 64),          # groups above 64 rows: chunks
    ([33, 1], 200, 768, 16),                # hint below the largest group
])
def test_grouped_matches_oracle(counts, N, K, hint):
    announce(f"w8a8_block_gemm_grouped counts={counts} N{N} K{K} hint{hint}")
    _run_and_check(counts, N, K, hint, seed=len(counts) + N)


def test_grouped_rows_outside_groups_untouched():
    announce("w8a8_block_gemm_grouped lead/tail rows")
    _run_and_check([4, 9, 0, 2], 160, 256, 16, seed=3, lead=5, tail=7)


@pytest.mark.parametrize("K,hint", [(6144, 64), (8192, 32)])
def test_grouped_long_k(K, hint):
    announce(f"w8a8_block_gemm_grouped long K{K} hint{hint}")
    _run_and_check([hint, 5, hint // 2], 256, K, hint, seed=K)


def test_grouped_all_experts_empty():
    announce("w8a8_block_gemm_grouped all experts empty")
    _run_and_check([0, 0, 0], 64, 128, 16, lead=3, tail=2)


def test_grouped_moe_decode_layer():
    cfg = workloads.MOE_DECODE
    counts = workloads.moe_routing(cfg["tokens"], cfg["E"], cfg["topk"], seed=0)
    announce(f"w8a8_block_gemm_grouped MoE decode E{cfg['E']} rows{int(counts.sum())} "
             f"N{cfg['N']} K{cfg['K']}")
    _run_and_check(counts, cfg["N"], cfg["K"], int(counts.max()), seed=0)
