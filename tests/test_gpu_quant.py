"""GPU parity of the four quantizers against the CPU oracle: bit-exact codes
and scales, through the C ABI (via the ctypes binding).

Cases: the 16 x 256 / 256 x 256 layer, ragged shapes (partial blocks,
K % 8 != 0, single rows), special blocks (all-zero, signed zeros,
saturating, bf16-max and bf16-subnormal amax, exact e4m3 blocks), every
finite bf16 pattern under a spread of block scales, and the full-size
weights and activations of the 7B / 32B-class layers (every byte and
scale of the whole arrays).  Output buffers carry canary
margins; repeated calls must give identical bits.
"""

import numpy as np
import pytest
import torch

from oracle import e4m3, quant
from precision_rl_rollout_amd import binding, workloads
from tests.gpu_util import Guarded, announce, bits_to_dev, host, oracle_by_rows

pytestmark = pytest.mark.gpu


def _fp8_w_gpu(w_bits):
    N, K = w_bits.shape
    q = Guarded((N, K), torch.uint8)
    s = Guarded((-(-N // 128), -(-K // 128)), torch.float32)
    binding.fp8_weight_block_quant(bits_to_dev(w_bits), out=q.t, scale=s.t)
    codes, scales = host(q.t), host(s.t)
    assert q.intact() and s.intact(), "write outside the output buffers"
    return codes, scales


def _fp8_a_gpu(a_bits):
    M, K = a_bits.shape
    q = Guarded((M, K), torch.uint8)
    s = Guarded((M, -(-K // 128)), torch.float32)
    binding.fp8_act_token_quant(bits_to_dev(a_bits), out=q.t, scale=s.t)
    codes, scales = host(q.t), host(s.t)
    assert q.intact() and s.intact(), "write outside the output buffers"
    return codes, scales


def _int8_gpu(fn, bits):
    R, K = bits.shape
    q = Guarded((R, K), torch.int8)
    s = Guarded((R,), torch.float32)
    fn(bits_to_dev(bits), out=q.t, scale=s.t)
    codes, scales = host(q.t), host(s.t)
    assert q.intact() and s.intact(), "write outside the output buffers"
    return codes, scales


def _same_f32_bits(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32),
                          np.asarray(b, np.float32).view(np.uint32))


def _assert_fp8_weight(w_bits, label):
    announce(f"fp8_weight_block_quant {label} {w_bits.shape}")
    codes, scales = _fp8_w_gpu(w_bits)
    rc, rs = quant.fp8_weight_block_quant(w_bits)
    assert _same_f32_bits(scales, rs), f"{label}: scales differ"
    bad = np.count_nonzero(codes != rc)
    assert bad == 0, f"{label}: {bad} code bytes differ"


def _assert_fp8_act(a_bits, label):
    announce(f"fp8_act_token_quant {label} {a_bits.shape}")
    codes, scales = _fp8_a_gpu(a_bits)
    rc, rs = quant.fp8_act_token_quant(a_bits)
    assert _same_f32_bits(scales, rs), f"{label}: scales differ"
    bad = np.count_nonzero(codes != rc)
    assert bad == 0, f"{label}: {bad} code bytes differ"


def _assert_int8(bits, label):
    for fn, ref in ((binding.int8_weight_channel_quant, quant.int8_weight_channel_quant),
                    (binding.int8_act_token_quant, quant.int8_act_token_quant)):
        announce(f"{fn.__name__} {label} {bits.shape}")
        codes, scales = _int8_gpu(fn, bits)
        rc, rs = ref(bits)
        assert _same_f32_bits(scales, rs), f"{label}: scales differ"
        assert np.array_equal(codes, rc), f"{label}: {np.count_nonzero(codes != rc)} codes differ"


# ----------------------------------------------------------------- shapes
SHAPES = [(256, 256), (16, 256), (300, 200), (130, 1000), (1, 129), (257, 385), (5, 37),
          (1, 1), (128, 8), (3, 4100), (1024, 1536)]


@pytest.mark.parametrize("shape", SHAPES)
def test_fp8_weight_quant_shapes(shape):
    for seed in (0, 1, 2):
        _assert_fp8_weight(workloads.weight(*shape, seed=seed), f"seed{seed}")


@pytest.mark.parametrize("shape", SHAPES)
def test_fp8_act_quant_shapes(shape):
    for seed in (0, 1, 2):
        _assert_fp8_act(workloads.activation(*shape, seed=seed, outliers=True), f"seed{seed}")


# Above 16 x 4 x 256 = 16,384 groups the activation quantizer gives each 16
# lanes four consecutive groups: K % 8 != 0 (per-element path) and == 0,
# groups per row not a multiple of four (runs that cross a row end), a
# ragged last workgroup.
ACT_LARGE = [(2100, 1001), (2050, 1160), (4099, 512)]


@pytest.mark.parametrize("shape", ACT_LARGE)
def test_fp8_act_quant_large_grids(shape):
    for seed in (0, 1):
        _assert_fp8_act(workloads.activation(*shape, seed=seed, outliers=True), f"seed{seed}")


@pytest.mark.parametrize("shape", SHAPES + [(64, 20000), (4, 40960), (3, 40963)])
def test_int8_quant_shapes(shape):
    for seed in (0, 1):
        _assert_int8(workloads.weight(*shape, seed=seed), f"seed{seed}")
        _assert_int8(workloads.activation(*shape, seed=seed, outliers=True), f"act seed{seed}")


# ----------------------------------------------------------------- special
def _special_matrix():
    """A 4 x 6 grid of 128 x 128 blocks with one special case per block."""
    rng = np.random.default_rng(123)
    w = workloads.weight(512, 768, seed=9)
    blocks = {}
    blocks[(0, 0)] = np.zeros((128, 128), np.uint16)                    # all +0
    z = np.zeros((128, 128), np.uint16)
    z[rng.random((128, 128)) < 0.5] = 0x8000
    blocks[(0, 1)] = z                                                  # signed zeros
    sign = (rng.integers(0, 2, (128, 128)).astype(np.uint16) << 15)
    blocks[(0, 2)] = sign | np.uint16(0x4234)                          # all +-45
    blocks[(0, 3)] = sign | np.uint16(0x7F7F)                          # all +-bf16 max
    blocks[(0, 4)] = sign | np.uint16(0x0001)                          # all +-min subnormal
    sub = rng.integers(0, 0x80, (128, 128)).astype(np.uint16) | sign   # bf16 subnormals
    blocks[(0, 5)] = sub
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    c = rng.choice(finite, size=(128, 128))
    c[3, 3] = 0x7E
    vals = e4m3.decode(c).astype(np.float32)
    blocks[(1, 0)] = (vals.view(np.uint32) >> 16).astype(np.uint16)    # exact e4m3, amax 448
    big = rng.integers(0x7000, 0x7F80, (128, 128)).astype(np.uint16) | sign
    blocks[(1, 1)] = big                                                # huge magnitudes
    one = np.zeros((128, 128), np.uint16)
    one[77, 5] = 0xBF80                                                 # a single -1.0
    blocks[(1, 2)] = one
    for (i, j), b in blocks.items():
        w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128] = b
    return w


def test_fp8_special_blocks():
    w = _special_matrix()
    _assert_fp8_weight(w, "special blocks")
    _assert_fp8_act(w, "special rows")
    codes, scales = _fp8_w_gpu(w)
    assert scales[0, 0] == 0 and scales[0, 1] == 0
    assert np.all(codes[:128, :128] == 0)
    assert np.array_equal(codes[:128, 128:256], np.where(w[:128, 128:256] != 0, 0x80, 0))
    for j in (2, 3, 4):
        blk = codes[:128, j * 128:(j + 1) * 128]
        assert np.all((blk & 0x7F) == 0x7E)
    assert scales[1, 0] == 1.0


def test_int8_special_rows():
    w = _special_matrix()
    _assert_int8(w, "special")


def _spread_of_scales():
    """64 blocks; block b has an amax drawn across the bf16 exponent range
    and holds random bf16 values of magnitude up to it, both signs."""
    rng = np.random.default_rng(77)
    amax_bits = np.unique(np.concatenate([
        rng.integers(0x0001, 0x7F80, 56), [0x0001, 0x0080, 0x3F80, 0x43E0, 0x7F7F, 0x0003,
                                           0x3C00, 0x4000]])).astype(np.uint16)[:64]
    blocks = []
    for ab in amax_bits:
        b = rng.integers(0, int(ab) + 1, (128, 128)).astype(np.uint16)
        b[0, 0] = ab
        b |= (rng.integers(0, 2, (128, 128)).astype(np.uint16) << 15)
        blocks.append(b)
    return np.concatenate(blocks, axis=0)


def test_fp8_all_bf16_patterns_and_scale_spread():
    w = _spread_of_scales()
    _assert_fp8_weight(w, "scale spread")
    _assert_fp8_act(w, "scale spread rows")
    pats = workloads.special_values_bf16()
    pats = np.concatenate([pats, np.zeros((-len(pats)) % (128 * 128), np.uint16)])
    grid = pats.reshape(-1, 128, 128).reshape(-1, 128)                 # sorted ranges per block
    _assert_fp8_weight(grid, "all finite bf16 patterns")
    _assert_fp8_act(grid, "all finite bf16 patterns as rows")
    rng = np.random.default_rng(3)
    _assert_fp8_weight(grid[rng.permutation(grid.shape[0])], "bf16 patterns shuffled rows")


def test_int8_all_bf16_patterns():
    pats = workloads.special_values_bf16()
    pats = np.concatenate([pats, np.zeros((-len(pats)) % 1024, np.uint16)]).reshape(-1, 1024)
    _assert_int8(pats, "all finite bf16 patterns")
    _assert_int8(_spread_of_scales(), "scale spread")


# ----------------------------------------------------------------- determinism
def test_repeat_calls_are_bitwise_identical():
    announce("determinism fp8/int8 quant 1024x1536")
    w = workloads.weight(1024, 1536, seed=5)
    a = _fp8_w_gpu(w)
    b = _fp8_w_gpu(w)
    assert np.array_equal(a[0], b[0]) and _same_f32_bits(a[1], b[1])
    c = _int8_gpu(binding.int8_weight_channel_quant, w)
    d = _int8_gpu(binding.int8_weight_channel_quant, w)
    assert np.array_equal(c[0], d[0]) and _same_f32_bits(c[1], d[1])


def test_empty_inputs():
    announce("empty quant inputs")
    for shape in ((0, 256), (5, 0), (0, 0)):
        t = torch.zeros(shape, dtype=torch.int16, device="cuda:0")
        q, s = binding.fp8_weight_block_quant(t)
        assert q.shape == shape
        q, s = binding.fp8_act_token_quant(t)
        q, s = binding.int8_weight_channel_quant(t)
        torch.cuda.synchronize()
        if shape[0]:
            assert torch.all(s == 0)


# ----------------------------------------------------------------- full size
# Whole arrays, every code byte and every scale bit, against the oracle run
# over row bands in parallel threads (the oracle's shard-commutation pin
# makes a band's result that part of the whole result).

def _assert_same(codes, scales, rc, rs, label):
    bad = int(np.count_nonzero(codes != rc))
    assert bad == 0, f"{label}: {bad} code bytes differ, first at {np.argwhere(codes != rc)[0]}"
    assert _same_f32_bits(scales, rs), f"{label}: scale bits differ"


def _full_fp8_weight(w, label):
    announce(f"fp8_weight_block_quant full-size {label} {w.shape}")
    codes, scales = _fp8_w_gpu(w)
    rc, rs = oracle_by_rows(quant.fp8_weight_block_quant, w, 1024)
    _assert_same(codes, scales, rc, rs, f"fp8 {label}")
    nb, kb = scales.shape
    # every block's largest code magnitude is 448 (0x7E), attained by its amax
    mx = (codes & 0x7F).reshape(nb, 128, kb, 128).max(axis=(1, 3))
    assert np.all(mx == 0x7E) and np.all(scales > 0)


def _full_int8(fn, ref, bits, label):
    announce(f"{fn.__name__} full-size {label} {bits.shape}")
    codes, scales = _int8_gpu(fn, bits)
    rc, rs = oracle_by_rows(ref, bits, 512)
    _assert_same(codes, scales, rc, rs, f"int8 {label}")
    assert np.all(np.abs(codes.astype(np.int32)).max(axis=1) == 127)


def test_full_size_7b_upgate_weight():
    w = workloads.weight(37888, 3584, seed=0)
    _full_fp8_weight(w, "7B up/gate")
    _full_int8(binding.int8_weight_channel_quant, quant.int8_weight_channel_quant, w,
               "7B up/gate")


@pytest.mark.parametrize("name", [n for n, _, _ in workloads.STACK_32B])
def test_full_size_32b_stack_weight(name):
    """Each of the seven weights of the 32B-class layer stack, FP8 blocks and
    INT8 channels, every byte and scale."""
    w = workloads.stack_layer(name, seed=0)
    _full_fp8_weight(w, f"32B {name}")
    _full_int8(binding.int8_weight_channel_quant, quant.int8_weight_channel_quant, w,
               f"32B {name}")


@pytest.mark.parametrize("K,stream", [(5120, "A"), (27648, "A_down")])
def test_full_size_32b_prefill_activations(K, stream):
    """All 8192 token rows of both prefill activations, FP8 groups and INT8
    rows."""
    a = workloads.activation(8192, K, seed=0, outliers=True, stream=stream)
    announce(f"fp8_act_token_quant full-size 32B prefill {a.shape}")
    codes, scales = _fp8_a_gpu(a)
    rc, rs = oracle_by_rows(quant.fp8_act_token_quant, a, 512)
    _assert_same(codes, scales, rc, rs, f"fp8 act K{K}")
    assert np.all((codes & 0x7F).reshape(8192, -1, 128).max(axis=2) == 0x7E)
    _full_int8(binding.int8_act_token_quant, quant.int8_act_token_quant, a, f"act K{K}")
