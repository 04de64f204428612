"""The allocation-free FP8 GEMM entry point (w8a8_block_gemm_scratch),
through the C ABI, against the entry point it varies (w8a8_block_gemm_ws
with a workspace of the size the library asks for): bit-identical outputs
on two calls in a row, the second with a smaller input, both within the
GEMM tolerance of the oracle; a shape whose split would need more than the
16 MiB static scratch is refused without a launch.
"""

import numpy as np
import pytest
import torch

from oracle import gemm, quant
from precision_rl_rollout_amd import binding, workloads
from tests.gpu_util import Guarded, announce, bits_to_dev, host

pytestmark = pytest.mark.gpu

SCRATCH = 16 << 20


def _operands(M, N, K, seed):
    p = workloads.gemm_problem(M, N, K, outliers=True, seed=seed, down=K > N)
    aq, sa = binding.fp8_act_token_quant(bits_to_dev(p["A"]))
    wq, sw = binding.fp8_weight_block_quant(bits_to_dev(p["Wt"]))
    return p, aq, sa, wq, sw


def _oracle_check(c, p):
    aq, sa = quant.fp8_act_token_quant(p["A"])
    wq, sw = quant.fp8_weight_block_quant(p["Wt"])
    ref = gemm.round_bf16(gemm.w8a8_block_gemm(aq, sa, wq, sw))
    err = gemm.rel_frobenius(c, ref)
    assert err <= 1e-3, err


def test_scratch_gemm_matches_the_workspace_call_twice():
    # The 32B down projection at a decode batch (split 5 ways, 6.5 MB of
    # partial sums), then a smaller split shape: the second call runs over
    # what the first left in the scratch.
    for M, N, K in ((64, 5120, 27648), (5, 300, 16384)):
        need = binding.gemm_workspace_bytes(M, N, K)
        assert 0 < need <= SCRATCH, (M, N, K, need)
        p, aq, sa, wq, sw = _operands(M, N, K, seed=M + N)
        announce(f"w8a8_block_gemm_scratch M{M} N{N} K{K} (split needs {need} B)")
        ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
        ref = host(binding.w8a8_block_gemm(aq, sa, wq, sw, workspace=ws))
        c = Guarded((M, N), torch.bfloat16)
        binding.w8a8_block_gemm_scratch(aq, sa, wq, sw, out=c.t)
        got = host(c.t)
        assert c.intact(), "write outside C"
        assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} outputs differ"
        _oracle_check(got, p)


def test_scratch_gemm_without_split_runs_one_pass():
    M, N, K = 64, 37888, 3584          # many strips: the one-pass kernel, no scratch
    assert binding.gemm_workspace_bytes(M, N, K) == 0
    p, aq, sa, wq, sw = _operands(M, N, K, seed=1)
    announce(f"w8a8_block_gemm_scratch one pass M{M} N{N} K{K}")
    ref = host(binding.w8a8_block_gemm(aq, sa, wq, sw, workspace=None))
    got = host(binding.w8a8_block_gemm_scratch(aq, sa, wq, sw))
    assert np.array_equal(got, ref)


def test_scratch_gemm_refuses_a_split_beyond_the_scratch():
    M, N, K = 64, 16384, 27648
    need = binding.gemm_workspace_bytes(M, N, K)
    assert need > SCRATCH, need
    announce(f"w8a8_block_gemm_scratch refused M{M} N{N} K{K} (split needs {need} B)")
    aq = torch.zeros((M, K), dtype=torch.uint8, device="cuda:0")
    sa = torch.zeros((M, K // 128), dtype=torch.float32, device="cuda:0")
    wq = torch.zeros((N, K), dtype=torch.uint8, device="cuda:0")
    sw = torch.zeros((N // 128, K // 128), dtype=torch.float32, device="cuda:0")
    c = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(binding.PrrError) as e:
        binding.w8a8_block_gemm_scratch(aq, sa, wq, sw, out=c)
    assert e.value.status == 2                     # PRR_ERR_UNSUPPORTED_SHAPE
    torch.cuda.synchronize()
    assert torch.all(c == 3.0)                     # nothing launched
