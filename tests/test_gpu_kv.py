"""GPU parity of the FP8 KV-cache calls against the oracle, bit for bit.

* fp8_kv_scale_recalibrate: the scale's bits, on ragged sizes (tails that are
  not whole 16-byte chunks), an all-zero and an empty tensor, values spread
  so the maximum sits in different workgroups, more chunks than one pass of
  the largest grid (threads loop), and the full 32B-layer size;
* fp8_kv_cache_write: every byte of the cache after the write, which covers
  the codes of written rows and the untouched rows (filled with a canary
  first), with padding and out-of-range slots, ragged C (per-element path),
  saturation beyond the calibrated range, a zero scale, and the full
  32B-layer prefill write.
"""

import numpy as np
import pytest
import torch

from oracle import kv
from precision_rl_rollout_amd import binding, workloads
from tests.gpu_util import announce, bits_to_dev, host

pytestmark = pytest.mark.gpu

CANARY = 0x5A


def _scale_gpu(xbits):
    return binding.fp8_kv_scale_recalibrate(bits_to_dev(xbits))


def _f32_bits(v) -> int:
    return int(np.asarray(v, dtype=np.float32).view(np.uint32))


@pytest.mark.parametrize("T,C", [(1, 1), (1, 7), (3, 5), (7, 40), (128, 1024), (333, 1001),
                                 (4096, 1024)])
def test_recalibrate_matches_oracle(T, C):
    for seed in (0, 1):
        xb = workloads.kv_rows(T, C, seed, "K")
        announce(f"fp8_kv_scale_recalibrate T{T} C{C} seed{seed}")
        got = host(_scale_gpu(xb))
        assert _f32_bits(got[0]) == _f32_bits(kv.kv_scale(xb))


def test_recalibrate_max_in_every_position():
    # one large value, moved through the first chunk, a middle chunk and the
    # ragged tail: every workgroup / tail path must see it
    T, C = 97, 123
    base = workloads.kv_rows(T, C, 4, "V")
    for pos in (0, 5, 8, T * C // 2, T * C - 8, T * C - 1):
        xb = base.copy().ravel()
        xb[pos] = 0xC3A0                        # -320.0
        xb = xb.reshape(T, C)
        announce(f"fp8_kv_scale_recalibrate max at {pos}")
        assert _f32_bits(host(_scale_gpu(xb))[0]) == _f32_bits(kv.kv_scale(xb))


def test_recalibrate_zero_and_empty():
    announce("fp8_kv_scale_recalibrate zero / empty")
    z = np.zeros((5, 64), dtype=np.uint16)
    z[2, 3] = 0x8000
    assert _f32_bits(host(_scale_gpu(z))[0]) == 0
    s = torch.full((1,), 7.0, device="cuda:0")
    e = torch.empty((0, 64), dtype=torch.int16, device="cuda:0")
    binding.fp8_kv_scale_recalibrate(e, out=s)
    torch.cuda.synchronize()
    assert _f32_bits(host(s)[0]) == 0


def test_recalibrate_past_one_pass_of_the_grid():
    # 66,000 x 1024 values: more 16-byte chunks than one pass of the grid
    # covers (one workgroup per CU, 32 chunks per thread: 2,097,152 chunks on
    # 256 CUs), so threads loop; the second check puts the maximum in the
    # last 11,000 chunks, which only the last pass reads
    T, C = 66000, 1024
    xb = workloads.kv_rows(T, C, 5, "K")
    announce(f"fp8_kv_scale_recalibrate T{T} C{C} (several passes)")
    xd = bits_to_dev(xb)
    assert _f32_bits(host(binding.fp8_kv_scale_recalibrate(xd))[0]) == _f32_bits(kv.kv_scale(xb))
    pos = T * C - 84_000
    xb.ravel()[pos] = 0xC4A0                    # -1280.0
    xd.view(-1)[pos] = int(np.int16(np.uint16(0xC4A0).view(np.int16)))
    assert _f32_bits(host(binding.fp8_kv_scale_recalibrate(xd))[0]) == _f32_bits(kv.kv_scale(xb))


def _write_case(T, C, num_slots, seed, pad_every=0, extra_slots=None, scale=None, xb=None):
    if xb is None:
        xb = workloads.kv_rows(T, C, seed, "V")
    slots = workloads.kv_slot_mapping(T, num_slots, 16, seed, pad_every)
    if extra_slots is not None:
        for t, sl in extra_slots.items():
            slots[t] = sl
    s = kv.kv_scale(xb) if scale is None else np.float32(scale)
    cache0 = np.full((num_slots, C), CANARY, dtype=np.uint8)
    want = kv.kv_cache_write(cache0, xb, slots, s)
    cache = torch.from_numpy(cache0).cuda()
    sd = torch.tensor([s], dtype=torch.float32, device="cuda:0")
    binding.fp8_kv_cache_write(bits_to_dev(xb), torch.from_numpy(slots).cuda(), sd, cache)
    return host(cache), want


@pytest.mark.parametrize("T,C,num_slots,pad", [(1, 8, 16, 0), (7, 40, 64, 3), (128, 1024, 512, 0),
                                               (333, 1001, 1024, 5), (100, 3, 2048, 0),
                                               (1000, 256, 4096, 9)])
def test_cache_write_matches_oracle(T, C, num_slots, pad):
    announce(f"fp8_kv_cache_write T{T} C{C} slots{num_slots} pad{pad}")
    got, want = _write_case(T, C, num_slots, seed=T + C, pad_every=pad)
    assert np.array_equal(got, want)


def test_cache_write_skips_out_of_range_slots():
    announce("fp8_kv_cache_write out-of-range slots")
    got, want = _write_case(40, 64, 128, seed=3,
                            extra_slots={0: -7, 5: 128, 6: 2 ** 40, 39: -(2 ** 62)})
    assert np.array_equal(got, want)


def test_cache_write_saturates_and_zero_scale():
    announce("fp8_kv_cache_write saturation / zero scale")
    xb = workloads.kv_rows(64, 128, 8, "K")
    small = np.float32(kv.kv_scale(xb) / 16)    # calibration range 16x too small
    got, want = _write_case(64, 128, 256, seed=8, scale=small, xb=xb)
    assert np.array_equal(got, want)
    assert np.count_nonzero((got == 0x7E) | (got == 0xFE)) > 0
    got, want = _write_case(64, 128, 256, seed=8, scale=0.0, xb=xb)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("scale", [2.0 ** -120 / 448, 2.0 ** -70, 2.0 ** -140, 1e-30, 2.0 ** -60])
def test_cache_write_stale_tiny_scale_saturates(scale):
    """A stale scale so small that x / s leaves the binary32 range (both the
    ordinary and the 2^96-prescaled division path): every such value
    saturates to +-448, the rest encode as usual."""
    announce(f"fp8_kv_cache_write stale tiny scale {scale:.3e}")
    xb = workloads.kv_rows(64, 128, 12, "K")
    xb[0, :8] = [0x3F80, 0xBF80, 0x0000, 0x8000, 0x0001, 0x8001, 0x7F7F, 0xFF7F]
    got, want = _write_case(64, 128, 256, seed=12, scale=np.float32(scale), xb=xb)
    assert np.array_equal(got, want)
    row0 = got[workloads.kv_slot_mapping(64, 256, 16, 12, 0)[0]]
    assert list(row0[[0, 1, 2, 3, 6, 7]]) == [0x7E, 0xFE, 0x00, 0x80, 0x7E, 0xFE]


def test_full_32b_prefill_write():
    cfg = workloads.KV_32B
    T, C, S = cfg["T"], cfg["C"], cfg["num_slots"]
    xb = workloads.kv_rows(T, C, 0, "K")
    announce(f"fp8_kv_scale_recalibrate + fp8_kv_cache_write full T{T} C{C} slots{S}")
    xd = bits_to_dev(xb)
    sd = binding.fp8_kv_scale_recalibrate(xd)
    s = kv.kv_scale(xb)
    assert _f32_bits(host(sd)[0]) == _f32_bits(s)
    slots = workloads.kv_slot_mapping(T, S, cfg["page"], 0)
    cache0 = np.full((S, C), CANARY, dtype=np.uint8)
    want = kv.kv_cache_write(cache0, xb, slots, s)
    cache = torch.from_numpy(cache0).cuda()
    binding.fp8_kv_cache_write(xd, torch.from_numpy(slots).cuda(), sd, cache)
    assert np.array_equal(host(cache), want)


# ------------------------------------------------- write + recalibrate, one pass
def _fused_case(T, C, num_slots, seed, pad_every=0, xb=None, stale_seed=None, inplace=False,
                workspace=None):
    """The step's rows written with the scale an earlier batch calibrated,
    and the next scale recalibrated from the same rows, in one call; the
    oracle's write and scale as the two steps.  inplace: the new scale
    replaces the old one in the same word."""
    if xb is None:
        xb = workloads.kv_rows(T, C, seed, "V")
    earlier = workloads.kv_rows(max(T, 1), max(C, 1), seed + 1000 if stale_seed is None
                                else stale_seed, "V")
    s_old = kv.kv_scale(earlier)
    slots = workloads.kv_slot_mapping(T, num_slots, 16, seed, pad_every) if T else \
        np.zeros(0, dtype=np.int64)
    cache0 = np.full((num_slots, C), CANARY, dtype=np.uint8)
    want_cache = kv.kv_cache_write(cache0, xb, slots, s_old) if T else cache0
    want_scale = kv.kv_scale(xb)
    cache = torch.from_numpy(cache0).cuda()
    sd = torch.tensor([s_old], dtype=torch.float32, device="cuda:0")
    new = sd if inplace else torch.full((1,), 7.0, dtype=torch.float32, device="cuda:0")
    binding.fp8_kv_cache_write_recalibrate(bits_to_dev(xb), torch.from_numpy(slots).cuda(), sd,
                                           cache, new_scale=new, workspace=workspace)
    return host(cache), host(new)[0], want_cache, want_scale, xb, slots, s_old


@pytest.mark.parametrize("T,C,num_slots,pad", [(1, 8, 16, 0), (7, 40, 64, 3), (128, 1024, 512, 0),
                                               (333, 1001, 1024, 5), (100, 3, 2048, 0),
                                               (1000, 256, 4096, 9)])
def test_write_recalibrate_matches_oracle(T, C, num_slots, pad):
    announce(f"fp8_kv_cache_write_recalibrate T{T} C{C} slots{num_slots} pad{pad}")
    got, got_s, want, want_s, *_ = _fused_case(T, C, num_slots, seed=T + C, pad_every=pad)
    assert np.array_equal(got, want)
    assert _f32_bits(got_s) == _f32_bits(want_s)


def test_write_recalibrate_in_place():
    # new_scale is the scale word: the rows are written with the old value,
    # then the word holds the new one.
    announce("fp8_kv_cache_write_recalibrate in place T300 C136")
    got, got_s, want, want_s, *_ = _fused_case(300, 136, 1024, seed=3, pad_every=4, inplace=True)
    assert np.array_equal(got, want)
    assert _f32_bits(got_s) == _f32_bits(want_s)


@pytest.mark.parametrize("T,C", [(20000, 1024), (600000, 8)])
def test_write_recalibrate_groups_past_the_grid(T, C):
    # More row groups than workgroups (2048): the workgroups loop; the
    # batch maximum sits in the last row, which a second pass reaches.
    xb = workloads.kv_rows(T, C, 41, "K")
    xb[T - 1, C - 1] = 0xC700                    # -32768.0
    announce(f"fp8_kv_cache_write_recalibrate T{T} C{C} (grid-stride)")
    got, got_s, want, want_s, *_ = _fused_case(T, C, T + 4096, seed=41, pad_every=13, xb=xb)
    assert np.array_equal(got, want)
    assert _f32_bits(got_s) == _f32_bits(want_s) == _f32_bits(np.float32(32768.0) / np.float32(448))


def test_write_recalibrate_reuses_a_workspace():
    # The partials of a large call are left in the workspace; a smaller
    # call on it reads only its own.
    ws = torch.empty(binding.KV_RECAL_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    big = workloads.kv_rows(16384, 256, 51, "K")
    big[100, 3] = 0x4780                         # 65536.0: a stale partial if read
    for T, C, xb in ((16384, 256, big), (9, 40, None), (1, 8, None)):
        announce(f"fp8_kv_cache_write_recalibrate T{T} C{C} on a used workspace")
        got, got_s, want, want_s, *_ = _fused_case(T, C, T + 64, seed=52, xb=xb, workspace=ws)
        assert np.array_equal(got, want)
        assert _f32_bits(got_s) == _f32_bits(want_s)


def test_write_recalibrate_counts_rows_without_a_slot():
    # The batch maximum sits in a padding row (negative slot): the write
    # skips the row, the scale counts it.
    T, C = 64, 128
    xb = workloads.kv_rows(T, C, 21, "K")
    slots_pad = workloads.kv_slot_mapping(T, 256, 16, 21, 7)
    pad_row = int(np.flatnonzero(slots_pad < 0)[0])
    xb[pad_row, 5] = 0x4700                      # 32768.0, far above the rest
    announce("fp8_kv_cache_write_recalibrate: maximum in a padding row")
    got, got_s, want, want_s, *_ = _fused_case(T, C, 256, seed=21, pad_every=7, xb=xb)
    assert np.array_equal(got, want)
    assert _f32_bits(got_s) == _f32_bits(want_s) == _f32_bits(np.float32(32768.0) / np.float32(448))


def test_write_recalibrate_equals_the_two_calls():
    T, C, S = 2000, 1024, 8192
    xb = workloads.kv_rows(T, C, 31, "K")
    slots = torch.from_numpy(workloads.kv_slot_mapping(T, S, 16, 31, 11)).cuda()
    xd = bits_to_dev(xb)
    s_old = binding.fp8_kv_scale_recalibrate(bits_to_dev(workloads.kv_rows(T, C, 32, "K")))
    announce("fp8_kv_cache_write_recalibrate against fp8_kv_cache_write + recalibrate")
    c1 = torch.full((S, C), CANARY, dtype=torch.uint8, device="cuda:0")
    c2 = c1.clone()
    binding.fp8_kv_cache_write(xd, slots, s_old, c1)
    s1 = binding.fp8_kv_scale_recalibrate(xd)
    s2 = binding.fp8_kv_cache_write_recalibrate(xd, slots, s_old, c2)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))


def test_write_recalibrate_empty_and_no_slots():
    announce("fp8_kv_cache_write_recalibrate: empty batch, empty cache")
    sd = torch.tensor([0.5], dtype=torch.float32, device="cuda:0")
    cache = torch.full((16, 8), CANARY, dtype=torch.uint8, device="cuda:0")
    empty = torch.empty((0, 8), dtype=torch.int16, device="cuda:0")
    new = binding.fp8_kv_cache_write_recalibrate(empty, torch.empty(0, dtype=torch.int64,
                                                                    device="cuda:0"), sd, cache)
    torch.cuda.synchronize()
    assert _f32_bits(host(new)[0]) == 0
    assert torch.all(cache == CANARY)
    # no cache rows at all: nothing written, the scale still recalibrated
    xb = workloads.kv_rows(9, 40, 5, "K")
    none = torch.empty((0, 40), dtype=torch.uint8, device="cuda:0")
    new = binding.fp8_kv_cache_write_recalibrate(
        bits_to_dev(xb), torch.arange(9, dtype=torch.int64, device="cuda:0"), sd, none)
    assert _f32_bits(host(new)[0]) == _f32_bits(kv.kv_scale(xb))


def test_full_32b_prefill_write_recalibrate():
    cfg = workloads.KV_32B
    T, C, S = cfg["T"], cfg["C"], cfg["num_slots"]
    announce(f"fp8_kv_cache_write_recalibrate full T{T} C{C} slots{S}")
    got, got_s, want, want_s, *_ = _fused_case(T, C, S, seed=0)
    assert np.array_equal(got, want)
    assert _f32_bits(got_s) == _f32_bits(want_s)


# ----------------------------------------- write + recalibrate, several tensors
def _multi_case(T, C, num_slots, seeds, pad_every=0, inplace=False):
    """Several tensors of one step (K, V, ...) sharing the slot mapping, in
    one fp8_kv_cache_write_recalibrate_multi call; each against the oracle's
    write with its earlier scale and its new scale."""
    slots = workloads.kv_slot_mapping(T, num_slots, 16, seeds[0], pad_every) if T else \
        np.zeros(0, dtype=np.int64)
    xs, olds, cache0s = [], [], []
    for i, sd in enumerate(seeds):
        xs.append(workloads.kv_rows(T, C, sd, "KV"[i % 2]))
        olds.append(kv.kv_scale(workloads.kv_rows(max(T, 1), max(C, 1), sd + 500, "KV"[i % 2])))
        cache0s.append(np.full((num_slots, C), CANARY, dtype=np.uint8))
    scales = [torch.tensor([s], dtype=torch.float32, device="cuda:0") for s in olds]
    caches = [torch.from_numpy(c).cuda() for c in cache0s]
    news = scales if inplace else None
    got_s = binding.fp8_kv_cache_write_recalibrate_multi(
        [bits_to_dev(x) for x in xs], torch.from_numpy(slots).cuda(), scales, caches,
        new_scales=news)
    for i in range(len(seeds)):
        want = kv.kv_cache_write(cache0s[i], xs[i], slots, olds[i]) if T else cache0s[i]
        assert np.array_equal(host(caches[i]), want), f"job {i}"
        assert _f32_bits(host(got_s[i])[0]) == _f32_bits(kv.kv_scale(xs[i])), f"job {i}"


@pytest.mark.parametrize("T,C,num_slots,pad", [(1, 8, 16, 0), (128, 1024, 512, 0),
                                               (333, 1001, 1024, 5), (1000, 256, 4096, 9)])
def test_write_recalibrate_multi_k_and_v(T, C, num_slots, pad):
    announce(f"fp8_kv_cache_write_recalibrate_multi K+V T{T} C{C} slots{num_slots} pad{pad}")
    _multi_case(T, C, num_slots, seeds=[T + 1, T + 2], pad_every=pad)


def test_write_recalibrate_multi_three_in_place():
    announce("fp8_kv_cache_write_recalibrate_multi 3 jobs in place T300 C136")
    _multi_case(300, 136, 1024, seeds=[7, 8, 9], pad_every=4, inplace=True)


def test_write_recalibrate_multi_equals_single_calls():
    T, C, S = 2000, 1024, 8192
    slots = torch.from_numpy(workloads.kv_slot_mapping(T, S, 16, 61, 11)).cuda()
    xk = bits_to_dev(workloads.kv_rows(T, C, 61, "K"))
    xv = bits_to_dev(workloads.kv_rows(T, C, 62, "V"))
    sk = binding.fp8_kv_scale_recalibrate(bits_to_dev(workloads.kv_rows(T, C, 63, "K")))
    sv = binding.fp8_kv_scale_recalibrate(bits_to_dev(workloads.kv_rows(T, C, 64, "V")))
    announce("fp8_kv_cache_write_recalibrate_multi against two single calls")
    ck1 = torch.full((S, C), CANARY, dtype=torch.uint8, device="cuda:0")
    cv1, ck2, cv2 = ck1.clone(), ck1.clone(), ck1.clone()
    nk1 = binding.fp8_kv_cache_write_recalibrate(xk, slots, sk, ck1)
    nv1 = binding.fp8_kv_cache_write_recalibrate(xv, slots, sv, cv1)
    nk2, nv2 = binding.fp8_kv_cache_write_recalibrate_multi([xk, xv], slots, [sk, sv], [ck2, cv2])
    torch.cuda.synchronize()
    assert torch.equal(ck1, ck2) and torch.equal(cv1, cv2)
    assert torch.equal(nk1.view(torch.int32), nk2.view(torch.int32))
    assert torch.equal(nv1.view(torch.int32), nv2.view(torch.int32))


def test_write_recalibrate_multi_empty_batch():
    announce("fp8_kv_cache_write_recalibrate_multi: empty batch")
    s = [torch.tensor([0.5], dtype=torch.float32, device="cuda:0") for _ in range(2)]
    caches = [torch.full((16, 8), CANARY, dtype=torch.uint8, device="cuda:0") for _ in range(2)]
    empty = torch.empty((0, 8), dtype=torch.int16, device="cuda:0")
    news = binding.fp8_kv_cache_write_recalibrate_multi(
        [empty, empty], torch.empty(0, dtype=torch.int64, device="cuda:0"), s, caches)
    torch.cuda.synchronize()
    assert all(_f32_bits(host(n)[0]) == 0 for n in news)
    assert all(bool(torch.all(c == CANARY)) for c in caches)


def test_full_32b_prefill_write_recalibrate_multi():
    cfg = workloads.KV_32B
    T, C, S = cfg["T"], cfg["C"], cfg["num_slots"]
    announce(f"fp8_kv_cache_write_recalibrate_multi full K+V T{T} C{C} slots{S}")
    _multi_case(T, C, S, seeds=[0, 1])
