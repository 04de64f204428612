"""GPU parity of fp8_weight_block_quant_into: shards of a weight quantized in
place into the full weight's code and scale arrays, against the CPU oracle.

* Tensor-parallel shards (rows of a column-parallel layer, columns of a
  row-parallel one, 128-aligned) assembled in a full buffer give exactly
  the oracle's quantization of the whole weight (codes and scales).
* Chunks read through strided views of the full bf16 weight on the device
  (row stride K, and a row stride that breaks 16-byte alignment, which takes
  the bounds-checked path) give the same.
* A ragged shard is quantized as a matrix of its own (the oracle on the
  sub-matrix) and nothing outside its rows, columns and scale blocks is
  written.
* Full size, in the launch configuration of the quantize-on-receive bench
  (the 32B up/gate weight in 8 chunks of 3456 rows through two staging
  buffers): equal to the whole-weight call, and to the oracle's
  quantization of the whole weight.
"""

import numpy as np
import pytest
import torch

from oracle import quant
from precision_rl_rollout_amd import binding, workloads
from tests.gpu_util import DEV, announce, bits_to_dev, host, oracle_by_rows

pytestmark = pytest.mark.gpu

CANARY = 0xA5


def _full_buffers(N, K):
    q = torch.full((N, K), CANARY, dtype=torch.uint8, device=DEV)
    s = torch.full((-(-N // 128), -(-K // 128)), float("nan"), dtype=torch.float32, device=DEV)
    return q, s


@pytest.mark.parametrize("N,K", [(1000, 1536), (512, 640)])
def test_tp_shards_assemble_the_full_quant(N, K):
    w = workloads.weight(N, K, seed=N + K)
    rq, rs = quant.fp8_weight_block_quant(w)
    wd = bits_to_dev(w)
    announce(f"fp8_weight_block_quant_into row shards {N}x{K}")
    q, s = _full_buffers(N, K)
    for r0 in range(0, N, 256):                        # column-parallel: rows
        binding.fp8_weight_block_quant_into(wd[r0:r0 + 256], q, s, row0=r0, col0=0)
    assert np.array_equal(host(q), rq) and np.array_equal(host(s), rs)
    announce(f"fp8_weight_block_quant_into column shards {N}x{K}")
    q, s = _full_buffers(N, K)
    step = 128 * max(1, K // 128 // 3)
    for c0 in range(0, K, step):                       # row-parallel: columns
        binding.fp8_weight_block_quant_into(wd[:, c0:c0 + step], q, s, row0=0, col0=c0)
    assert np.array_equal(host(q), rq) and np.array_equal(host(s), rs)


def test_unaligned_row_stride_takes_the_checked_path():
    N, K = 384, 512
    w = workloads.weight(N, K, seed=3)
    rq, rs = quant.fp8_weight_block_quant(w)
    wide = np.zeros((N, K + 3), dtype=np.uint16)       # row stride K + 3 elements
    wide[:, :K] = w
    wd = bits_to_dev(wide)[:, :K]
    announce("fp8_weight_block_quant_into row stride K + 3")
    q, s = _full_buffers(N, K)
    for r0 in (0, 128, 256):
        binding.fp8_weight_block_quant_into(wd[r0:r0 + 128], q, s, row0=r0, col0=0)
    assert np.array_equal(host(q), rq) and np.array_equal(host(s), rs)


def test_ragged_shard_writes_only_its_own_blocks():
    N, K = 512, 1024
    r0, c0, rows, cols = 128, 256, 200, 300
    sub = workloads.weight(rows, cols, seed=11)
    rq, rs = quant.fp8_weight_block_quant(sub)
    announce("fp8_weight_block_quant_into ragged 200x300 shard at (128, 256)")
    q, s = _full_buffers(N, K)
    binding.fp8_weight_block_quant_into(bits_to_dev(sub), q, s, row0=r0, col0=c0)
    hq, hs = host(q), host(s)
    assert np.array_equal(hq[r0:r0 + rows, c0:c0 + cols], rq)
    outside = np.ones((N, K), dtype=bool)
    outside[r0:r0 + rows, c0:c0 + cols] = False
    assert (hq[outside] == CANARY).all()
    b0, bc0 = r0 // 128, c0 // 128
    assert np.array_equal(hs[b0:b0 + rs.shape[0], bc0:bc0 + rs.shape[1]], rs)
    so = np.ones(hs.shape, dtype=bool)
    so[b0:b0 + rs.shape[0], bc0:bc0 + rs.shape[1]] = False
    assert np.isnan(hs[so]).all()


def test_full_size_32b_upgate_in_eight_chunks():
    N, K, chunks = 27648, 5120, 8
    rows = N // chunks
    w = workloads.weight(N, K, seed=0)
    wd = bits_to_dev(w)
    announce("fp8_weight_block_quant_into full-size 32B up/gate, 8 chunks")
    q, s = _full_buffers(N, K)
    stage = [torch.empty((rows, K), dtype=torch.int16, device=DEV) for _ in range(2)]
    for c in range(chunks):
        buf = stage[c % 2]
        buf.copy_(wd[c * rows:(c + 1) * rows])
        binding.fp8_weight_block_quant_into(buf, q, s, row0=c * rows)
    wq, ws = binding.fp8_weight_block_quant(wd)
    hq, hs = host(q), host(s)
    assert np.array_equal(hq, host(wq)) and np.array_equal(hs.view(np.uint32), host(ws).view(np.uint32))
    rq, rs = oracle_by_rows(quant.fp8_weight_block_quant, w, 1024)
    assert np.array_equal(hq, rq)
    assert np.array_equal(hs.view(np.uint32), rs.view(np.uint32))
