"""Seeded sweeps of the remaining calls against the CPU oracle through the
C ABI.

* TIS / MIS token weights (tis_token_weights): 12 draws (seed 13) of 1-40
  sequences of 1-5000 token positions, both modes, a cap drawn from
  1.01-4, padding poisoned with NaN and infinities; counts and cap
  decisions exact, weights and sums within the bounds test_gpu_tis.py
  uses.
* Quantize-on-receive (fp8_weight_block_quant_into): 10 draws (seed 17) of
  a full weight up to 1000 x 2000 and a ragged shard at a random
  128-aligned offset inside it; the shard's codes and scales must equal the
  oracle's quantization of the shard, byte for byte and bit for bit, and
  nothing outside its blocks may change.
* One-launch stack quantization (fp8_weight_block_quant_multi,
  int8_weight_channel_quant_multi): 4 draws (seed 19) of 1-16 ragged weights
  (one possibly empty); every weight's codes and scales as the oracle's.
"""

import numpy as np
import pytest
import torch

from oracle import quant, tis
from precision_rl_rollout_amd import binding, workloads
from tests.gpu_util import DEV, announce, bits_to_dev, host
from tests.test_gpu_quant_multi import _same_bits
from tests.test_gpu_tis import _check as _tis_check
from tests.test_gpu_tis import _poison_padding
from tests.test_gpu_tis import _run as _tis_run

pytestmark = pytest.mark.gpu

CANARY = 0xA5


def _tis_draws(seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 41)), int(rng.integers(1, 5001)),
             float(np.float32(rng.uniform(1.01, 4.0))), i) for i in range(12)]


def _into_draws(seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(10):
        N, K = int(rng.integers(1, 1001)), int(rng.integers(1, 2001))
        r0 = 128 * int(rng.integers(0, -(-N // 128)))
        c0 = 128 * int(rng.integers(0, -(-K // 128)))
        rows = int(rng.integers(1, N - r0 + 1))
        cols = int(rng.integers(1, K - c0 + 1))
        out.append((N, K, r0, c0, rows, cols, i))
    return out


def _multi_draws(seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(4):
        n = int(rng.integers(1, 17))
        shapes = [(int(rng.integers(0 if j == 0 else 1, 600)), int(rng.integers(1, 3000)))
                  for j in range(n)]
        out.append((tuple(shapes), i))
    return out


@pytest.mark.parametrize("B,T,cap,i", _tis_draws(13))
def test_tis_sweep(B, T, cap, i):
    p = _poison_padding(workloads.tis_batch(B, T, seed=100 + i), seed=i)
    for mode in (tis.TRUNCATE, tis.MASK):
        announce(f"tis_token_weights sweep #{i}: B{B} T{T} cap{cap:.4f} mode{mode}")
        _tis_check(p, cap, mode, _tis_run(p, cap, mode), f"sweep #{i} mode{mode}")


@pytest.mark.parametrize("N,K,r0,c0,rows,cols,i", _into_draws(17))
def test_quant_into_sweep(N, K, r0, c0, rows, cols, i):
    announce(f"fp8_weight_block_quant_into sweep #{i}: {rows}x{cols} shard at ({r0}, {c0}) "
             f"of {N}x{K}")
    sub = workloads.weight(rows, cols, seed=200 + i)
    rq, rs = quant.fp8_weight_block_quant(sub)
    q = torch.full((N, K), CANARY, dtype=torch.uint8, device=DEV)
    s = torch.full((-(-N // 128), -(-K // 128)), float("nan"), dtype=torch.float32, device=DEV)
    binding.fp8_weight_block_quant_into(bits_to_dev(sub), q, s, row0=r0, col0=c0)
    hq, hs = host(q), host(s)
    assert np.array_equal(hq[r0:r0 + rows, c0:c0 + cols], rq)
    outside = np.ones((N, K), dtype=bool)
    outside[r0:r0 + rows, c0:c0 + cols] = False
    assert (hq[outside] == CANARY).all()
    b0, bc0 = r0 // 128, c0 // 128
    assert _same_bits(hs[b0:b0 + rs.shape[0], bc0:bc0 + rs.shape[1]], rs)
    so = np.ones(hs.shape, dtype=bool)
    so[b0:b0 + rs.shape[0], bc0:bc0 + rs.shape[1]] = False
    assert np.isnan(hs[so]).all()


@pytest.mark.parametrize("shapes,i", _multi_draws(19))
def test_multi_quant_sweep(shapes, i):
    announce(f"fp8/int8 multi-weight quant sweep #{i}: {len(shapes)} weights")
    ws = [workloads.weight(N, K, seed=300 + 17 * i + j) for j, (N, K) in enumerate(shapes)]
    devs = [bits_to_dev(w) for w in ws]
    got8 = binding.fp8_weight_block_quant_multi(devs)
    goti = binding.int8_weight_channel_quant_multi(devs)
    for w, (q8, s8), (qi, si), shape in zip(ws, got8, goti, shapes):
        rc, rs = quant.fp8_weight_block_quant(w)
        assert np.array_equal(host(q8), rc) and _same_bits(host(s8), rs), ("fp8", shape)
        rc, rs = quant.int8_weight_channel_quant(w)
        assert np.array_equal(host(qi), rc) and _same_bits(host(si), rs), ("int8", shape)
