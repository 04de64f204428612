"""GPU parity of the multi-weight re-quantization calls
(fp8_weight_block_quant_multi, int8_weight_channel_quant_multi), through the
C ABI: every code byte and scale bit equal to the oracle's on ragged weights
of every row class, and equal to the one-weight calls on the full 32B-class
layer stack (whose one-weight results are compared with the oracle in full
by test_gpu_quant.py)."""

import numpy as np
import pytest
import torch

from oracle import quant
from precision_rl_rollout_amd import binding, workloads
from tests.gpu_util import announce, bits_to_dev, host

pytestmark = pytest.mark.gpu

# Partial blocks, K % 8 != 0, and INT8 rows of all three classes (a wave per
# row up to K 8192, a workgroup per row up to 32768, two passes beyond or
# with K % 8 != 0), one empty job.
RAGGED = [(300, 200), (1, 129), (257, 385), (5, 37), (128, 8192), (130, 8200), (3, 40960),
          (2, 40963), (0, 128), (1024, 1536), (7, 1)]


def _same_bits(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32),
                          np.asarray(b, np.float32).view(np.uint32))


def test_multi_ragged_against_the_oracle():
    ws = [workloads.weight(N, K, seed=i) for i, (N, K) in enumerate(RAGGED)]
    devs = [bits_to_dev(w) for w in ws]
    announce(f"fp8/int8 multi-weight quant, {len(ws)} ragged weights")
    got8 = binding.fp8_weight_block_quant_multi(devs)
    goti = binding.int8_weight_channel_quant_multi(devs)
    for w, (q8, s8), (qi, si), shape in zip(ws, got8, goti, RAGGED):
        rc, rs = quant.fp8_weight_block_quant(w)
        assert np.array_equal(host(q8), rc) and _same_bits(host(s8), rs), ("fp8", shape)
        rc, rs = quant.int8_weight_channel_quant(w)
        assert np.array_equal(host(qi), rc) and _same_bits(host(si), rs), ("int8", shape)


def test_multi_32b_stack_equals_one_call_per_weight():
    devs = [bits_to_dev(workloads.stack_layer(n, seed=0)) for n, _, _ in workloads.STACK_32B]
    announce("fp8/int8 multi-weight quant of the 32B layer stack (7 weights)")
    multi8 = binding.fp8_weight_block_quant_multi(devs)
    multii = binding.int8_weight_channel_quant_multi(devs)
    for (name, _, _), w, (q8, s8), (qi, si) in zip(workloads.STACK_32B, devs, multi8, multii):
        r8, rs8 = binding.fp8_weight_block_quant(w)
        ri, rsi = binding.int8_weight_channel_quant(w)
        torch.cuda.synchronize()
        assert torch.equal(q8, r8) and torch.equal(s8.view(torch.int32), rs8.view(torch.int32)), name
        assert torch.equal(qi, ri) and torch.equal(si.view(torch.int32), rsi.view(torch.int32)), name


def test_multi_empty_and_repeat():
    announce("multi-weight quant: empty list, repeatability")
    assert binding.fp8_weight_block_quant_multi([]) == []
    w = bits_to_dev(workloads.weight(640, 1000, seed=4))
    a = binding.fp8_weight_block_quant_multi([w, w])
    torch.cuda.synchronize()
    assert torch.equal(a[0][0], a[1][0]) and torch.equal(a[0][1], a[1][1])


def test_multi_at_the_job_limit():
    # As many weights as one launch takes (the job table travels in the
    # kernel arguments), the last job's blocks at the end of the grid.
    shapes = [(64 + 37 * i, 128 + 61 * i) for i in range(binding.MAX_WEIGHT_JOBS)]
    ws = [workloads.weight(N, K, seed=100 + i) for i, (N, K) in enumerate(shapes)]
    devs = [bits_to_dev(w) for w in ws]
    announce(f"fp8/int8 multi-weight quant, {len(ws)} weights (the job limit)")
    got8 = binding.fp8_weight_block_quant_multi(devs)
    goti = binding.int8_weight_channel_quant_multi(devs)
    for w, (q8, s8), (qi, si), shape in zip(ws, got8, goti, shapes):
        rc, rs = quant.fp8_weight_block_quant(w)
        assert np.array_equal(host(q8), rc) and _same_bits(host(s8), rs), ("fp8", shape)
        rc, rs = quant.int8_weight_channel_quant(w)
        assert np.array_equal(host(qi), rc) and _same_bits(host(si), rs), ("int8", shape)
