"""A seeded sweep of ragged quantizer shapes, bit-exact against the CPU
oracle through the C ABI: FP8 128 x 128 weight blocks, FP8 1 x 128
activation groups, INT8 per-channel weights and INT8 per-token activations.

The fixed shape lists elsewhere pin the workloads' layers and chosen edge
cases; this sweep draws 20 shapes per quantizer (seed 7) with rows from 1
to 700 and K from 1 to 9000, so that partial blocks and groups, K not a
multiple of 8 (the element-wise paths) and K a multiple of 8 (the 16-byte
paths) all appear, and zeroes one random block or row in every other case
(the all-zero scale).  Codes must match byte for byte and scales bit for
bit; every output sits in a guard band that must stay untouched.
"""

import numpy as np
import pytest

from oracle import quant
from precision_rl_rollout_amd import binding, workloads
from tests.gpu_util import announce
from tests.test_gpu_quant import _fp8_a_gpu, _fp8_w_gpu, _int8_gpu, _same_f32_bits

pytestmark = pytest.mark.gpu


def _shapes(seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(20):
        R = int(rng.integers(1, 701))
        K = int(rng.integers(1, 9001))
        if i % 3 == 0:
            K = max(8, K // 8 * 8)          # a multiple of 8: the vector paths
        out.append((R, K, i % 2 == 1))
    return out


SHAPES = _shapes(7)


def _input(R, K, zero, weight):
    bits = (workloads.weight(R, K, seed=R * 7 + K) if weight
            else workloads.activation(R, K, seed=R * 7 + K))
    if zero:
        rng = np.random.default_rng(R + K)
        if weight:   # one whole 128 x 128 block (partial at the edges)
            r0 = 128 * int(rng.integers(0, -(-R // 128)))
            c0 = 128 * int(rng.integers(0, -(-K // 128)))
            bits[r0:r0 + 128, c0:c0 + 128] = 0
        else:        # one whole row
            bits[int(rng.integers(0, R))] = 0
    return bits


def _assert_same(codes, scales, ref, label):
    rc, rs = ref
    assert _same_f32_bits(scales, rs), f"{label}: scales differ"
    bad = np.count_nonzero(codes != rc)
    assert bad == 0, f"{label}: {bad} code bytes differ"


@pytest.mark.parametrize("R,K,zero", SHAPES)
def test_fp8_weight_sweep(R, K, zero):
    announce(f"fp8 weight quant sweep {R}x{K} zero={zero}")
    w = _input(R, K, zero, True)
    _assert_same(*_fp8_w_gpu(w), quant.fp8_weight_block_quant(w), f"fp8 W {R}x{K}")


@pytest.mark.parametrize("R,K,zero", SHAPES)
def test_fp8_act_sweep(R, K, zero):
    announce(f"fp8 act quant sweep {R}x{K} zero={zero}")
    a = _input(R, K, zero, False)
    _assert_same(*_fp8_a_gpu(a), quant.fp8_act_token_quant(a), f"fp8 A {R}x{K}")


@pytest.mark.parametrize("R,K,zero", SHAPES)
def test_int8_weight_sweep(R, K, zero):
    announce(f"int8 weight quant sweep {R}x{K} zero={zero}")
    w = _input(R, K, zero, True)
    _assert_same(*_int8_gpu(binding.int8_weight_channel_quant, w),
                 quant.int8_weight_channel_quant(w), f"int8 W {R}x{K}")


@pytest.mark.parametrize("R,K,zero", SHAPES)
def test_int8_act_sweep(R, K, zero):
    announce(f"int8 act quant sweep {R}x{K} zero={zero}")
    a = _input(R, K, zero, False)
    _assert_same(*_int8_gpu(binding.int8_act_token_quant, a),
                 quant.int8_act_token_quant(a), f"int8 A {R}x{K}")
