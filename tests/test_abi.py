"""The C ABI of libprr.so, checked from the host (no kernel is launched).

* the library loads and exports every function ``include/prr.h`` declares;
* every argument check returns its documented status before any device
  work (negative / oversized dimensions, NULL and misaligned pointers,
  unsupported GEMM shapes); empty calls succeed and touch nothing;
* without a visible device, a well-formed call returns PRR_ERR_NO_DEVICE.

Pointers passed here are never dereferenced: every call fails (or is empty)
before the library reaches a launch -- in a process without a GPU, where a
well-formed call stops at the device check.  With a GPU visible those calls
would launch kernels on the fake addresses, so the whole module is skipped
there (it belongs to the CPU suite).
"""

import ctypes
import os
import re

import pytest

from precision_rl_rollout_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "prr.h")

OK, INVALID, SHAPE, MISALIGNED, NO_DEVICE, BAD_DEVICE, HIP = range(7)
FAKE = 0x10000          # 16-byte aligned, never dereferenced
ODD = 0x10008           # 8-byte aligned only


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:prr_status|const char\*|int)\s+(\w+)\s*\(", text, flags=re.M)


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


pytestmark = pytest.mark.skipif(
    _gpu_visible(), reason="passes fake device pointers through the argument checks; a "
                           "process with a GPU would launch kernels on them")


def test_header_declares_the_boundary():
    names = set(_declared())
    assert names == {"fp8_weight_block_quant", "fp8_weight_block_quant_into",
                     "fp8_act_token_quant", "w8a8_block_gemm",
                     "int8_weight_channel_quant", "int8_act_token_quant",
                     "w8a8_int8_channel_gemm", "w8a8_block_gemm_grouped",
                     "fp8_kv_scale_recalibrate",
                     "fp8_kv_cache_write", "fp8_kv_cache_write_recalibrate",
                     "tis_token_weights", "w8a8_gemm_workspace_size",
                     "fp8_kv_decode_attention", "fp8_kv_decode_attention_workspace_size",
                     "fp8_kv_decode_attention_ws", "w8a8_block_gemm_ws",
                     "w8a8_int8_channel_gemm_ws", "w8a8_block_gemm_scratch",
                     "fp8_weight_block_quant_multi", "int8_weight_channel_quant_multi",
                     "fp8_kv_cache_write_recalibrate_multi",
                     "prr_status_string", "prr_abi_version"}


def test_library_exports_every_declared_symbol():
    lib = binding.load()
    for name in _declared():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    header = open(HEADER).read()
    declared = int(re.search(r"#define PRR_ABI_VERSION (\d+)", header).group(1))
    assert binding.abi_version() == declared == binding.ABI_VERSION
    names = [binding.status_string(s) for s in range(7)]
    assert names == ["PRR_OK", "PRR_ERR_INVALID_ARG", "PRR_ERR_UNSUPPORTED_SHAPE",
                     "PRR_ERR_MISALIGNED", "PRR_ERR_NO_DEVICE", "PRR_ERR_UNSUPPORTED_DEVICE",
                     "PRR_ERR_HIP"]
    assert binding.status_string(99) == "PRR_ERR_UNKNOWN"


QUANTS = ["fp8_weight_block_quant", "fp8_act_token_quant", "int8_weight_channel_quant",
          "int8_act_token_quant"]
GEMMS = ["w8a8_block_gemm", "w8a8_int8_channel_gemm", "w8a8_block_gemm_scratch"]


@pytest.mark.parametrize("fn", QUANTS)
def test_quant_argument_checks(fn):
    c = lambda *a: binding.call(fn, *a)
    assert c(FAKE, -1, 128, FAKE, FAKE, None) == INVALID
    assert c(FAKE, 128, -5, FAKE, FAKE, None) == INVALID
    assert c(FAKE, 2 ** 31, 128, FAKE, FAKE, None) == INVALID
    assert c(None, 4, 128, FAKE, FAKE, None) == INVALID
    assert c(FAKE, 4, 128, None, FAKE, None) == INVALID
    assert c(FAKE, 4, 128, FAKE, None, None) == INVALID
    assert c(ODD, 4, 128, FAKE, FAKE, None) == MISALIGNED
    assert c(FAKE, 4, 128, ODD, FAKE, None) == MISALIGNED
    assert c(FAKE, 4, 128, FAKE, ODD, None) == MISALIGNED
    # empty along the leading dimension: nothing to do, NULLs allowed
    assert c(None, 0, 128, None, None, None) == OK


@pytest.mark.parametrize("fn", ["fp8_weight_block_quant", "fp8_act_token_quant"])
def test_fp8_quant_empty_k_is_a_no_op(fn):
    assert binding.call(fn, None, 7, 0, None, None, None) == OK


@pytest.mark.parametrize("fn", GEMMS)
def test_gemm_argument_checks(fn):
    c = lambda *a: binding.call(fn, *a)
    P = [FAKE] * 4
    assert c(*P, -1, 16, 128, FAKE, None) == INVALID
    assert c(*P, 1, -16, 128, FAKE, None) == INVALID
    assert c(*P, 1, 16, -128, FAKE, None) == INVALID
    assert c(*P, 1, 16, 100, FAKE, None) == SHAPE
    assert c(*P, 1, 16, 129, FAKE, None) == SHAPE
    for i in range(4):
        q = list(P)
        q[i] = None
        assert c(*q, 1, 16, 128, FAKE, None) == INVALID
        q[i] = ODD
        assert c(*q, 1, 16, 128, FAKE, None) == MISALIGNED
    assert c(*P, 1, 16, 128, None, None) == INVALID
    assert c(*P, 1, 16, 128, ODD, None) == MISALIGNED
    assert c(None, None, None, None, 0, 16, 128, None, None) == OK
    assert c(None, None, None, None, 5, 0, 128, None, None) == OK


def test_int8_gemm_rejects_k_that_could_overflow_int32():
    P = [FAKE] * 4
    K = 133248            # first multiple of 128 above 133143
    assert binding.call("w8a8_int8_channel_gemm", *P, 1, 16, K, FAKE, None) == SHAPE
    if not _gpu_visible():
        # the FP8 GEMM has no such limit: it gets as far as the device check
        # (skipped where a device exists, since that call would launch)
        assert binding.call("w8a8_block_gemm", *P, 1, 16, K, FAKE, None) == NO_DEVICE


@pytest.mark.parametrize("fn", GEMMS + ["w8a8_block_gemm_ws", "w8a8_int8_channel_gemm_ws"])
def test_gemm_rejects_k_beyond_the_tile_offsets(fn):
    """K above 65535 blocks is refused before any device work, for every
    dense GEMM call (the last accepted K, 8388480, reaches the device check
    in a process without a GPU)."""
    P = [FAKE] * 4
    ws = (None, 0) if fn.endswith("_ws") else ()
    assert binding.call(fn, *P, 65, 16, 8388608, FAKE, *ws, None) == SHAPE
    assert binding.call(fn, *P, 1, 16, 8388480 + 128, FAKE, *ws, None) == SHAPE
    if not _gpu_visible() and not fn.startswith("w8a8_int8"):
        assert binding.call(fn, *P, 65, 16, 8388480, FAKE, *ws, None) == NO_DEVICE


@pytest.mark.skipif(_gpu_visible(), reason="needs a process without a GPU")
@pytest.mark.parametrize("fn", QUANTS + GEMMS)
def test_no_device_is_reported(fn):
    if fn in GEMMS:
        st = binding.call(fn, FAKE, FAKE, FAKE, FAKE, 16, 256, 256, FAKE, None)
    else:
        st = binding.call(fn, FAKE, 16, 256, FAKE, FAKE, None)
    assert st == NO_DEVICE


def test_kv_recalibrate_argument_checks():
    c = lambda *a: binding.call("fp8_kv_scale_recalibrate", *a)
    assert c(FAKE, -1, 8, FAKE, None) == INVALID
    assert c(FAKE, 8, 2 ** 31, FAKE, None) == INVALID
    assert c(None, 4, 8, FAKE, None) == INVALID
    assert c(FAKE, 4, 8, None, None) == INVALID
    assert c(ODD, 4, 8, FAKE, None) == MISALIGNED
    assert c(FAKE, 4, 8, ODD, None) == MISALIGNED
    # an empty tensor still writes its scale (0): the output pointer is needed
    assert c(None, 0, 8, None, None) == INVALID


def test_kv_cache_write_argument_checks():
    c = lambda *a: binding.call("fp8_kv_cache_write", *a)
    assert c(FAKE, FAKE, -1, 8, FAKE, FAKE, 4, None) == INVALID
    assert c(FAKE, FAKE, 4, 8, FAKE, FAKE, -4, None) == INVALID
    for i in (0, 1, 4, 5):
        args = [FAKE, FAKE, 4, 8, FAKE, FAKE, 16, None]
        args[i] = None
        assert c(*args) == INVALID
        args[i] = ODD
        assert c(*args) == MISALIGNED
    # nothing to write: no pointer is needed
    assert c(None, None, 0, 8, None, None, 16, None) == OK
    assert c(None, None, 4, 0, None, None, 16, None) == OK
    assert c(None, None, 4, 8, None, None, 0, None) == OK


def test_kv_write_recalibrate_argument_checks():
    c = lambda *a: binding.call("fp8_kv_cache_write_recalibrate", *a)
    NEW = FAKE + 256                             # another aligned word
    WS = FAKE + 4096
    WSB = binding.KV_RECAL_WORKSPACE_BYTES
    assert WSB == 8192
    assert c(FAKE, FAKE, -1, 8, FAKE, FAKE, 4, NEW, WS, WSB, None) == INVALID
    assert c(FAKE, FAKE, 4, 8, FAKE, FAKE, -4, NEW, WS, WSB, None) == INVALID
    assert c(FAKE, FAKE, 4, 8, FAKE, FAKE, 16, NEW, WS, -1, None) == INVALID
    for i in (0, 1, 4, 5, 7, 8):
        args = [FAKE, FAKE, 4, 8, FAKE, FAKE, 16, NEW, WS, WSB, None]
        args[i] = None
        assert c(*args) == INVALID, i
        args[i] = ODD
        assert c(*args) == MISALIGNED, i
    # the partial maxima need the whole workspace
    assert c(FAKE, FAKE, 4, 8, FAKE, FAKE, 16, NEW, WS, WSB - 4, None) == INVALID
    # an empty batch still writes its new scale (0): that pointer is needed
    assert c(None, None, 0, 8, None, None, 16, None, None, 0, None) == INVALID


@pytest.mark.skipif(_gpu_visible(), reason="needs a process without a GPU")
def test_kv_no_device_is_reported():
    assert binding.call("fp8_kv_scale_recalibrate", FAKE, 4, 8, FAKE, None) == NO_DEVICE
    assert binding.call("fp8_kv_cache_write", FAKE, FAKE, 4, 8, FAKE, FAKE, 16, None) == NO_DEVICE
    WSB = binding.KV_RECAL_WORKSPACE_BYTES
    assert binding.call("fp8_kv_cache_write_recalibrate", FAKE, FAKE, 4, 8, FAKE, FAKE, 16,
                        FAKE + 256, FAKE + 4096, WSB, None) == NO_DEVICE
    # the new scale may be the scale word (updated in place)
    assert binding.call("fp8_kv_cache_write_recalibrate", FAKE, FAKE, 4, 8, FAKE, FAKE, 16,
                        FAKE, FAKE + 4096, WSB, None) == NO_DEVICE
    # an empty batch or no slots: nothing is read (no workspace either), the
    # new scale is still set
    assert binding.call("fp8_kv_cache_write_recalibrate", None, None, 0, 8, None, None, 16,
                        FAKE, None, 0, None) == NO_DEVICE
    assert binding.call("fp8_kv_cache_write_recalibrate", FAKE, FAKE, 4, 8, FAKE, None, 0,
                        FAKE + 256, FAKE + 4096, WSB, None) == NO_DEVICE


def test_tis_argument_checks():
    c = lambda *a: binding.call("tis_token_weights", *a)
    ok = [FAKE, FAKE, FAKE, 4, 8, 2.0, 0, FAKE, FAKE, FAKE, None]
    bad = dict(B=(3, -1), T=(4, -8), cap0=(5, 0.0), capneg=(5, -1.0), capnan=(5, float("nan")),
               mode=(6, 2))
    for _, (i, v) in bad.items():
        a = list(ok)
        a[i] = v
        assert c(*a) == INVALID
    for i in (0, 1, 2, 7):
        a = list(ok)
        a[i] = None
        assert c(*a) == INVALID
        a[i] = ODD
        assert c(*a) == MISALIGNED
    a = list(ok)
    a[8] = None                                  # totals need the row statistics
    assert c(*a) == INVALID
    a = list(ok)
    a[4] = 2 ** 24 + 4                           # counts must stay exact in fp32
    assert c(*a) == SHAPE
    # nothing to compute and nothing to report: no pointer is needed
    assert c(None, None, None, 0, 8, 2.0, 1, None, None, None, None) == OK
    assert c(None, None, None, 4, 0, 2.0, 0, None, None, None, None) == OK


@pytest.mark.skipif(_gpu_visible(), reason="needs a process without a GPU")
def test_tis_no_device_is_reported():
    assert binding.call("tis_token_weights", FAKE, FAKE, FAKE, 4, 8, 2.0, 0, FAKE, FAKE, FAKE,
                        None) == NO_DEVICE
    assert binding.call("tis_token_weights", None, None, None, 0, 8, 2.0, 0, None, None, FAKE,
                        None) == NO_DEVICE


@pytest.mark.parametrize("fn", ["w8a8_block_gemm_ws", "w8a8_int8_channel_gemm_ws"])
def test_gemm_ws_argument_checks(fn):
    c = lambda *a: binding.call(fn, *a)
    ok = [FAKE, FAKE, FAKE, FAKE, 16, 256, 256, FAKE, FAKE, 1024, None]
    for i, v in ((4, -1), (5, -2), (6, -128), (9, -1)):
        a = list(ok)
        a[i] = v
        assert c(*a) == INVALID
    a = list(ok)
    a[6] = 200
    assert c(*a) == SHAPE
    for i in (0, 1, 2, 3, 7):
        a = list(ok)
        a[i] = None
        assert c(*a) == INVALID
        a[i] = ODD
        assert c(*a) == MISALIGNED
    a = list(ok)
    a[8] = ODD                                   # a workspace must be aligned too
    assert c(*a) == MISALIGNED
    assert c(None, None, None, None, 0, 256, 256, None, None, 0, None) == OK


def test_workspace_size_argument_checks():
    n = ctypes.c_int64(-1)
    c = lambda *a: binding.call("w8a8_gemm_workspace_size", *a)
    assert c(4, 8, 256, None) == INVALID
    assert c(-1, 8, 256, ctypes.addressof(n)) == INVALID
    assert c(4, 8, 200, ctypes.addressof(n)) == SHAPE
    assert c(0, 8, 256, ctypes.addressof(n)) == OK and n.value == 0


def test_attention_argument_checks():
    c = lambda *a: binding.call("fp8_kv_decode_attention", *a)
    ok = [FAKE] * 8 + [4, 40, 8, 128, 16, 64, 4096, 0.088, FAKE, None]
    for i, v in ((8, -1), (9, -1), (10, -1), (12, -16), (13, -1), (14, -1),
                 (15, float("nan")), (15, float("inf"))):
        a = list(ok)
        a[i] = v
        assert c(*a) == INVALID, (i, v)
    for i, v in ((11, 64), (9, 41), (9, 80), (10, 3)):
        a = list(ok)
        a[i] = v
        assert c(*a) == SHAPE, (i, v)
    for i in (0, 1, 2, 3, 4, 5, 6, 7, 16):
        a = list(ok)
        a[i] = None
        assert c(*a) == INVALID
        a[i] = ODD
        assert c(*a) == MISALIGNED
    a = list(ok)
    a[12] = 0                                    # a page of zero tokens
    assert c(*a) == INVALID
    # nothing to compute: no pointer is needed
    assert c(*([None] * 8 + [0, 40, 8, 128, 16, 64, 4096, 0.088, None, None])) == OK


def test_attention_ws_argument_checks():
    c = lambda *a: binding.call("fp8_kv_decode_attention_ws", *a)
    ok = [FAKE] * 8 + [4, 40, 8, 128, 16, 64, 4096, 0.088, FAKE, FAKE, 1 << 20, None]
    a = list(ok)
    a[18] = -1                                   # negative workspace size
    assert c(*a) == INVALID
    for i, v in ((8, -1), (10, -1), (15, float("nan"))):
        a = list(ok)
        a[i] = v
        assert c(*a) == INVALID, (i, v)
    for i, v in ((11, 64), (9, 41)):
        a = list(ok)
        a[i] = v
        assert c(*a) == SHAPE, (i, v)
    a = list(ok)
    a[17] = ODD                                  # a misaligned workspace
    assert c(*a) == MISALIGNED
    for i in (0, 6, 16):
        a = list(ok)
        a[i] = None
        assert c(*a) == INVALID
    # nothing to compute: no pointer is needed
    assert c(*([None] * 8 + [0, 40, 8, 128, 16, 64, 4096, 0.088, None, None, 0, None])) == OK
    n = ctypes.c_int64(-1)
    z = lambda *a: binding.call("fp8_kv_decode_attention_workspace_size", *a)
    assert z(4, 40, 8, 128, None) == INVALID
    assert z(-1, 40, 8, 128, ctypes.addressof(n)) == INVALID
    assert z(0, 40, 8, 128, ctypes.addressof(n)) == OK and n.value == 0


def test_quant_into_argument_checks():
    c = lambda *a: binding.call("fp8_weight_block_quant_into", *a)
    ok = [FAKE, 256, 384, 512, FAKE, 1024, FAKE, 8, None]
    for i, v in ((1, -1), (2, -5), (3, 383), (5, 100), (7, 2), (3, -1)):
        a = list(ok)
        a[i] = v
        assert c(*a) == INVALID, (i, v)
    for i in (0, 4, 6):
        a = list(ok)
        a[i] = None
        assert c(*a) == INVALID
    a = list(ok)
    a[0] = ODD
    assert c(*a) == MISALIGNED
    a = list(ok)
    a[6] = FAKE + 2                              # scales need 4-byte alignment only
    assert c(*a) == MISALIGNED
    a = list(ok)
    a[6] = FAKE + 4
    assert c(*a) == NO_DEVICE
    assert c(*ok) == NO_DEVICE
    assert c(None, 0, 384, 0, None, 0, None, 0, None) == OK      # empty: nothing touched


@pytest.mark.parametrize("fn", ["fp8_weight_block_quant_multi", "int8_weight_channel_quant_multi"])
def test_multi_weight_argument_checks(fn):
    J = binding.WeightJob
    c = lambda jobs, n: binding.call(fn, None if jobs is None else ctypes.addressof(jobs), n, None)
    one = (J * 1)(J(FAKE, 4, 128, FAKE, FAKE))
    assert c(None, 0) == OK                               # nothing to do
    assert c(None, 1) == INVALID                          # jobs missing
    assert c(one, -1) == INVALID
    assert c(one, binding.MAX_WEIGHT_JOBS + 1) == INVALID
    for bad, want in ((J(FAKE, -1, 128, FAKE, FAKE), INVALID), (J(FAKE, 4, 2 ** 31, FAKE, FAKE), INVALID),
                      (J(None, 4, 128, FAKE, FAKE), INVALID), (J(FAKE, 4, 128, None, FAKE), INVALID),
                      (J(FAKE, 4, 128, FAKE, None), INVALID), (J(ODD, 4, 128, FAKE, FAKE), MISALIGNED),
                      (J(FAKE, 4, 128, ODD, FAKE), MISALIGNED), (J(FAKE, 4, 128, FAKE, ODD), MISALIGNED)):
        two = (J * 2)(J(FAKE, 4, 128, FAKE, FAKE), bad)
        assert c(two, 2) == want
    empty = (J * 2)(J(None, 0, 128, None, None), J(None, 0, 0, None, None))
    assert c(empty, 2) == OK                              # empty jobs: no device work
    if not _gpu_visible():
        assert c(one, 1) == NO_DEVICE


def test_kv_write_recalibrate_multi_argument_checks():
    J = binding.KvJob
    WSB = binding.KV_RECAL_WORKSPACE_BYTES
    c = lambda jobs, n, T=4, C=8, S=16, ws=FAKE + 8192, wsb=2 * WSB: binding.call(
        "fp8_kv_cache_write_recalibrate_multi", None if jobs is None else ctypes.addressof(jobs),
        n, FAKE, T, C, S, ws, wsb, None)
    good = lambda k: J(FAKE + 16 * k, FAKE + 256 + 16 * k, FAKE + 512 + 16 * k, FAKE + 1024 + 16 * k)
    two = (J * 2)(good(0), good(1))
    assert binding.MAX_KV_JOBS == 16
    assert c(None, 0) == OK                                # nothing to do
    assert c(None, 1) == INVALID                           # jobs missing
    assert c(two, -1) == INVALID
    assert c(two, binding.MAX_KV_JOBS + 1) == INVALID
    assert c(two, 2, T=-1) == INVALID
    assert c(two, 2, wsb=2 * WSB - 4) == INVALID           # a workspace slot per job
    assert c(two, 2, ws=None) == INVALID
    assert c(two, 2, ws=ODD) == MISALIGNED
    for field in ("kv_bf16", "scale", "cache", "new_scale"):
        for v, want in ((None, INVALID), (ODD, MISALIGNED)):
            bad = good(1)
            setattr(bad, field, v)
            assert c((J * 2)(good(0), bad), 2) == want, (field, v)
    dup = good(1)
    dup.new_scale = good(0).new_scale                      # the new scales must be distinct
    assert c((J * 2)(good(0), dup), 2) == INVALID
    if not _gpu_visible():
        assert c(two, 2) == NO_DEVICE
        # a new scale may be its own job's scale word (updated in place)
        inplace = good(0)
        inplace.new_scale = inplace.scale
        assert c((J * 1)(inplace), 1, wsb=WSB) == NO_DEVICE
        # an empty batch: rows, caches and workspace unused; the new scales are set
        empty = (J * 2)(J(None, None, None, FAKE), J(None, None, None, FAKE + 16))
        assert c(empty, 2, T=0, ws=None, wsb=0) == NO_DEVICE
