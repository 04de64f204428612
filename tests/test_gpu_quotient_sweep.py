"""The division and conversion shortcuts of the quantizers, swept through
the C ABI against the oracle, byte for byte.

The kernels do not divide every element by the block scale s with a full
IEEE division and do not build e4m3 codes with integer arithmetic: they form
r = RN(1 / s) once per block, correct each quotient with one fused
multiply-add (Markstein's step; blocks with s < 2^-64 first scale x and s by
2^96), and convert with the hardware fp32 -> e4m3 instruction.  The
definition is encode(fl32(x / s)).  This test feeds the library's own
quantizers blocks built so that, for every amax value of a set, every finite
bf16 x with |x| <= amax (both signs, and both zeros) is divided by
s = fl32(amax / 448) (FP8) or fl32(amax / 127) (INT8), and compares every
code with the oracle's.

The amax set covers every bf16 binade: in each of the 254 normal binades the
power of two, 448 * 2^k (s is then an exact power of two, the quotients are
exact and every e4m3 midpoint among them is a tie), the largest mantissa and
a seeded random mantissa; plus 16 subnormal amax values (the 2^96 path is
taken for every amax below 448 * 2^-64, about 70 binades).  1,031 amax
values in all (one random mantissa repeats), about 34 million (x, s) pairs
per quantizer.

The FP8-KV write with s = 1 divides exactly (r = 1, the correction adds
zero), so its codes are the conversion of every finite bf16 value itself:
the hardware conversion against the oracle's bit-built encoder on all of
them, saturation above 448 included.
"""

import numpy as np
import pytest
import torch

from oracle import kv, quant
from precision_rl_rollout_amd import binding
from tests.gpu_util import Guarded, announce, bits_to_dev, host, oracle_by_rows, u8_to_dev

pytestmark = pytest.mark.gpu


def amax_set() -> np.ndarray:
    rng = np.random.default_rng(20250)
    vals = []
    for ef in range(1, 255):
        for mant in (0x00, 0x60, 0x7F, int(rng.integers(1, 0x7F))):
            vals.append((ef << 7) | mant)
    vals += [0x0001, 0x0002, 0x0003, 0x007F]
    vals += [int(v) for v in rng.choice(np.arange(4, 0x7F), 12, replace=False)]
    return np.unique(np.array(vals, dtype=np.uint16))


def _pieces(group: int) -> np.ndarray:
    """Rows of `group` bf16 values: each row starts with its amax and holds a
    run of the bf16 values of magnitude <= amax (both signs; zeros pad)."""
    rows = []
    for a in amax_set():
        mags = np.arange(0, int(a) + 1, dtype=np.uint16)
        xs = np.concatenate([mags, mags | np.uint16(0x8000)])
        per = group - 1
        n = -(-len(xs) // per)
        pad = np.zeros(n * per, np.uint16)
        pad[:len(xs)] = xs
        body = pad.reshape(n, per)
        rows.append(np.concatenate([np.full((n, 1), a, np.uint16), body], axis=1))
    return np.concatenate(rows, axis=0)


def test_amax_set_covers_every_binade():
    a = amax_set()
    assert len(a) >= 1000
    assert set(range(1, 255)) <= set(int(v) >> 7 for v in a)
    assert np.any(a < 0x80)                                       # subnormal amax
    ties = (a & 0x7F) == 0x60                                     # 448 * 2^k
    assert ties.sum() == 254
    # the tiny-scale path is taken below 448 * 2^-64
    s = (a.astype(np.uint32) << 16).view(np.float32) / np.float32(448)
    assert np.count_nonzero(s < np.float32(2.0 ** -64)) > 200


def test_fp8_weight_blocks_sweep():
    rows = _pieces(128 * 128).reshape(-1, 128)            # one 128 x 128 block per piece
    announce(f"fp8_weight_block_quant quotient sweep {rows.shape}")
    q = Guarded(rows.shape, torch.uint8)
    s = Guarded((rows.shape[0] // 128, 1), torch.float32)
    binding.fp8_weight_block_quant(bits_to_dev(rows), out=q.t, scale=s.t)
    codes, scales = host(q.t), host(s.t)
    assert q.intact() and s.intact()
    rc, rs = oracle_by_rows(quant.fp8_weight_block_quant, rows, 128 * 64)
    assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32))
    bad = np.count_nonzero(codes != rc)
    assert bad == 0, f"{bad} codes differ, first at {np.argwhere(codes != rc)[0]}"


def test_fp8_act_groups_sweep():
    groups = _pieces(128)
    groups = np.concatenate([groups, np.zeros(((-len(groups)) % 64, 128), np.uint16)])
    rows = groups.reshape(-1, 128 * 64)                   # 64 groups per token row
    announce(f"fp8_act_token_quant quotient sweep {rows.shape}")
    codes, scales = (host(t) for t in binding.fp8_act_token_quant(bits_to_dev(rows)))
    rc, rs = oracle_by_rows(quant.fp8_act_token_quant, rows, 2048)
    assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32))
    assert np.count_nonzero(codes != rc) == 0


@pytest.mark.parametrize("K", [4096, 16384])
def test_int8_rows_sweep(K):
    rows = _pieces(K)
    announce(f"int8_weight_channel_quant quotient sweep {rows.shape}")
    codes, scales = (host(t) for t in binding.int8_weight_channel_quant(bits_to_dev(rows)))
    rc, rs = oracle_by_rows(quant.int8_weight_channel_quant, rows, 256)
    assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32))
    assert np.count_nonzero(codes != rc) == 0


def test_fp8_conversion_of_every_bf16_value():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF].reshape(-1, 128)      # finite patterns
    T, C = bits.shape
    announce(f"fp8_kv_cache_write s=1 conversion of every finite bf16 {bits.shape}")
    one = torch.ones(1, dtype=torch.float32, device="cuda:0")
    cache = u8_to_dev(np.zeros((T, C), np.uint8))
    slots = torch.arange(T, dtype=torch.int64, device="cuda:0")
    binding.fp8_kv_cache_write(bits_to_dev(bits), slots, one, cache)
    got = host(cache)
    ref = kv.kv_encode_rows(bits, np.float32(1.0))
    assert np.count_nonzero(got != ref) == 0
