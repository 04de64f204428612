"""Seeded sweeps of two more calls against the CPU oracle through the C ABI.

* The FP8 KV cache write with recalibration in one pass
  (fp8_kv_cache_write_recalibrate): 16 draws (seed 5) of tokens T 1-3000,
  channels C 1-2048, a cache of the pages T needs plus 0-199 spare ones,
  and padding (rows without a slot) every 0-9 tokens; every cache byte and
  the new scale's bits must equal the oracle's write with the old scale and
  its recalibration from the same rows.
* The grouped MoE GEMM (w8a8_block_gemm_grouped): 12 draws (seed 9) of 1-40
  experts with 0-80 rows each (a third of them empty), N 1-700, K 1-24
  blocks, the row-count hint at, below or above the largest group, and
  leading and trailing rows outside every group (which must stay
  untouched); the bar is the one test_gpu_gemm_grouped.py uses.
"""

import numpy as np
import pytest

from tests.gpu_util import announce
from tests.test_gpu_gemm_grouped import _run_and_check
from tests.test_gpu_kv import _f32_bits, _fused_case

pytestmark = pytest.mark.gpu


def _kv_draws(seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(16):
        T = int(rng.integers(1, 3001))
        C = int(rng.integers(1, 2049))
        slots = 16 * (-(-T // 16) + int(rng.integers(0, 200)))   # the pages T needs, plus spare
        pad = int(rng.integers(0, 10))
        out.append((T, C, slots, pad))
    return out


def _moe_draws(seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(12):
        E = int(rng.integers(1, 41))
        counts = [0 if rng.random() < 1 / 3 else int(rng.integers(1, 81)) for _ in range(E)]
        N = int(rng.integers(1, 701))
        K = 128 * int(rng.integers(1, 25))
        top = max(counts) if max(counts) > 0 else 16
        hint = int(rng.choice([top, max(1, top // 2), 64]))
        lead, tail = int(rng.integers(0, 5)), int(rng.integers(0, 5))
        out.append((tuple(counts), N, K, hint, lead, tail, i))
    return out


@pytest.mark.parametrize("T,C,num_slots,pad", _kv_draws(5))
def test_kv_write_recalibrate_sweep(T, C, num_slots, pad):
    announce(f"fp8_kv_cache_write_recalibrate sweep T{T} C{C} slots{num_slots} pad{pad}")
    got, got_s, want, want_s, *_ = _fused_case(T, C, num_slots, seed=T * 3 + C, pad_every=pad)
    assert np.array_equal(got, want)
    assert _f32_bits(got_s) == _f32_bits(want_s)


@pytest.mark.parametrize("counts,N,K,hint,lead,tail,i", _moe_draws(9))
def test_grouped_gemm_sweep(counts, N, K, hint, lead, tail, i):
    announce(f"w8a8_block_gemm_grouped sweep #{i}: E{len(counts)} rows {sum(counts)} N{N} K{K} "
             f"hint{hint} lead{lead} tail{tail}")
    _run_and_check(list(counts), N, K, hint, seed=i, lead=lead, tail=tail)
