"""Thin ctypes binding over libprr.so.

Every function here has the name of the C entry point it calls (see
``include/prr.h``) and does argument marshalling only: it checks dtypes,
shapes and devices of torch tensors, allocates the outputs with torch on the
input's device, passes raw pointers and the current HIP stream, and raises
``PrrError`` on a non-OK status.  All arithmetic happens in the HIP kernels.
Calls with an optional workspace (the GEMMs and the decode attention) take
``workspace="auto"`` (a buffer of the size the library asks for, the
default), ``None`` (the calls without one) or a uint8 CUDA tensor.

bf16 inputs may be ``torch.bfloat16`` or ``torch.int16`` / ``torch.uint16``
tensors holding bf16 bit patterns.  FP8 outputs are ``torch.uint8`` codes
(OCP e4m3; ``.view(torch.float8_e4m3fn)`` reinterprets them), INT8 outputs
``torch.int8``, scales ``torch.float32``, GEMM outputs ``torch.bfloat16``.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PRR_LIB may point the binding at another build of the same library (the
# CPU tests load a host-AddressSanitizer build of the ABI layer this way).
LIB_PATH = os.environ.get("PRR_LIB") or os.path.join(_HERE, "libprr.so")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64

_SIGNATURES = {
    "fp8_weight_block_quant": [_P, _I64, _I64, _P, _P, _P],
    "fp8_weight_block_quant_into": [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P],
    "fp8_act_token_quant": [_P, _I64, _I64, _P, _P, _P],
    "w8a8_block_gemm": [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P],
    "int8_weight_channel_quant": [_P, _I64, _I64, _P, _P, _P],
    "int8_act_token_quant": [_P, _I64, _I64, _P, _P, _P],
    "w8a8_int8_channel_gemm": [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P],
    "w8a8_block_gemm_grouped": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P],
    "fp8_kv_scale_recalibrate": [_P, _I64, _I64, _P, _P],
    "fp8_kv_cache_write": [_P, _P, _I64, _I64, _P, _P, _I64, _P],
    "tis_token_weights": [_P, _P, _P, _I64, _I64, ctypes.c_float, ctypes.c_int, _P, _P, _P, _P],
    "w8a8_gemm_workspace_size": [_I64, _I64, _I64, _P],
    "fp8_kv_decode_attention": [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                _I64, _I64, ctypes.c_float, _P, _P],
    "fp8_kv_decode_attention_workspace_size": [_I64, _I64, _I64, _I64, _P],
    "fp8_kv_decode_attention_ws": [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                   _I64, _I64, ctypes.c_float, _P, _P, _I64, _P],
    "w8a8_block_gemm_ws": [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I64, _P],
    "w8a8_int8_channel_gemm_ws": [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I64, _P],
    "w8a8_block_gemm_scratch": [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P],
    "fp8_kv_cache_write_recalibrate": [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _I64, _P],
    "fp8_kv_cache_write_recalibrate_multi": [_P, _I64, _P, _I64, _I64, _I64, _P, _I64, _P],
    "fp8_weight_block_quant_multi": [_P, _I64, _P],
    "int8_weight_channel_quant_multi": [_P, _I64, _P],
}

MAX_WEIGHT_JOBS = 16
MAX_KV_JOBS = 16


class WeightJob(ctypes.Structure):
    """prr_weight_job: one whole weight and its outputs."""
    _fields_ = [("w_bf16", _P), ("N", _I64), ("K", _I64), ("q", _P), ("scale", _P)]

class KvJob(ctypes.Structure):
    """prr_kv_job: one tensor of a step's KV cache write + recalibration."""
    _fields_ = [("kv_bf16", _P), ("scale", _P), ("cache", _P), ("new_scale", _P)]

IS_TRUNCATE = 0     # TIS: min(ratio, cap)
IS_MASK = 1         # MIS: ratio, or 0 above the cap

_lib = None

# PRR_ABI_VERSION of the signatures below; a library of another version is
# refused at load time.
ABI_VERSION = 11


class PrrError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} ({status})")


def load() -> ctypes.CDLL:
    """Load libprr.so (once).  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m precision_rl_rollout_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.prr_status_string.argtypes = [ctypes.c_int]
        lib.prr_status_string.restype = ctypes.c_char_p
        lib.prr_abi_version.argtypes = []
        lib.prr_abi_version.restype = ctypes.c_int
        if lib.prr_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {lib.prr_abi_version()}, the "
                               f"binding expects {ABI_VERSION}; rebuild it")
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().prr_status_string(int(status)).decode()


def abi_version() -> int:
    return load().prr_abi_version()


def call(name: str, *args) -> int:
    """Call a C entry point with raw arguments; returns its status."""
    return getattr(load(), name)(*args)


def _stream(t: torch.Tensor) -> int:
    # The library runs on the current HIP device (its checks, launches and
    # per-device scratch all follow it): the tensors must live there.
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"tensor on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}; call under "
                         f"torch.cuda.device({t.device.index})")
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: torch.Tensor | None):
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _check(name: str, status: int) -> None:
    if status != 0:
        raise PrrError(name, status)


def _bf16_bits(t: torch.Tensor, what: str) -> torch.Tensor:
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{what}: expected bf16 (or int16 bit patterns), got {t.dtype}")
    if not t.is_cuda or t.dim() != 2 or not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous 2-D CUDA tensor")
    return t


def _operand(t: torch.Tensor, dtype, shape, what: str) -> torch.Tensor:
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_cuda \
            or not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous CUDA {dtype} tensor of shape "
                         f"{tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    return t


def _out(out, dtype, shape, like: torch.Tensor, what: str) -> torch.Tensor:
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    return _operand(out, dtype, shape, what)


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def fp8_weight_block_quant(w: torch.Tensor, out=None, scale=None):
    """Wt [N, K] bf16 -> (codes uint8 [N, K], scales fp32 [ceil(N/128), ceil(K/128)])."""
    w = _bf16_bits(w, "w")
    N, K = w.shape
    q = _out(out, torch.uint8, (N, K), w, "out")
    s = _out(scale, torch.float32, (_cdiv(N, 128), _cdiv(K, 128)), w, "scale")
    _check("fp8_weight_block_quant",
           load().fp8_weight_block_quant(_ptr(w), N, K, _ptr(q), _ptr(s), _stream(w)))
    return q, s


def fp8_weight_block_quant_into(w: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                                row0: int = 0, col0: int = 0):
    """Quantize the bf16 shard w [rows, cols] (any row stride, unit column
    stride) into rows row0.. and columns col0.. of a full weight's codes
    uint8 [N, K] and scales fp32 [ceil(N/128), ceil(K/128)]; row0 and col0
    are multiples of 128 (the shard's blocks are then the full weight's)."""
    if w.dtype not in (torch.bfloat16, torch.int16) or not w.is_cuda or w.dim() != 2:
        raise ValueError("w: expected a 2-D CUDA bf16 tensor")
    if w.shape[1] > 1 and w.stride(1) != 1:
        raise ValueError("w: columns must be contiguous")
    if row0 % 128 or col0 % 128 or row0 < 0 or col0 < 0:
        raise ValueError("row0 and col0 must be non-negative multiples of 128")
    rows, cols = w.shape
    N, K = codes.shape
    _operand(codes, torch.uint8, (N, K), "codes")
    _operand(scales, torch.float32, (_cdiv(N, 128), _cdiv(K, 128)), "scales")
    if row0 + rows > N or col0 + cols > K:
        raise ValueError("the shard does not fit the full weight at (row0, col0)")
    if rows == 0 or cols == 0:
        return codes, scales
    _check("fp8_weight_block_quant_into",
           load().fp8_weight_block_quant_into(
               w.data_ptr(), rows, cols, w.stride(0), codes.data_ptr() + row0 * K + col0, K,
               scales.data_ptr() + 4 * ((row0 // 128) * scales.shape[1] + col0 // 128),
               scales.shape[1], _stream(w)))
    return codes, scales


def fp8_act_token_quant(a: torch.Tensor, out=None, scale=None):
    """A [M, K] bf16 -> (codes uint8 [M, K], scales fp32 [M, ceil(K/128)])."""
    a = _bf16_bits(a, "a")
    M, K = a.shape
    q = _out(out, torch.uint8, (M, K), a, "out")
    s = _out(scale, torch.float32, (M, _cdiv(K, 128)), a, "scale")
    _check("fp8_act_token_quant",
           load().fp8_act_token_quant(_ptr(a), M, K, _ptr(q), _ptr(s), _stream(a)))
    return q, s


_ws_sizes: dict = {}


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace (bytes) the _ws GEMM calls use for this shape on the current
    device; 0 when the one-pass kernels are used.  (Remembered per device
    and shape: the answer depends only on them.)"""
    key = (torch.cuda.current_device(), int(M), int(N), int(K))
    if key not in _ws_sizes:
        n = ctypes.c_int64(0)
        _check("w8a8_gemm_workspace_size",
               load().w8a8_gemm_workspace_size(int(M), int(N), int(K), ctypes.addressof(n)))
        _ws_sizes[key] = int(n.value)
    return _ws_sizes[key]


def _workspace(workspace, M, N, K, like):
    """workspace="auto": a buffer of the size the library asks for (none if
    it asks for none); None: no workspace; a uint8 CUDA tensor: used as is."""
    if workspace is None:
        return None
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace: 'auto', None or a uint8 CUDA tensor")
        n = gemm_workspace_bytes(M, N, K) if M > 0 and N > 0 and K > 0 else 0
        return torch.empty((n,), dtype=torch.uint8, device=like.device) if n else None
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace: expected a contiguous CUDA uint8 tensor")
    return workspace


def w8a8_block_gemm(a_fp8, a_scale, w_fp8, w_scale, out=None, workspace="auto"):
    """FP8 codes + block scales -> C [M, N] bf16.  With a workspace (by
    default one of the size the library asks for), decode-sized batches of
    narrow or long-K layers, and the last partial round of a many-token
    long-K layer, are split over K (w8a8_block_gemm_ws)."""
    M, K = a_fp8.shape
    N = w_fp8.shape[0]
    _operand(a_fp8, torch.uint8, (M, K), "a_fp8")
    _operand(w_fp8, torch.uint8, (N, K), "w_fp8")
    _operand(a_scale, torch.float32, (M, _cdiv(K, 128)), "a_scale")
    _operand(w_scale, torch.float32, (_cdiv(N, 128), _cdiv(K, 128)), "w_scale")
    c = _out(out, torch.bfloat16, (M, N), a_fp8, "out")
    ws = _workspace(workspace, M, N, K, a_fp8)
    if ws is None:
        _check("w8a8_block_gemm",
               load().w8a8_block_gemm(_ptr(a_fp8), _ptr(a_scale), _ptr(w_fp8), _ptr(w_scale),
                                      M, N, K, _ptr(c), _stream(a_fp8)))
    else:
        _check("w8a8_block_gemm_ws",
               load().w8a8_block_gemm_ws(_ptr(a_fp8), _ptr(a_scale), _ptr(w_fp8), _ptr(w_scale),
                                         M, N, K, _ptr(c), _ptr(ws), ws.numel(), _stream(a_fp8)))
    return c


def w8a8_block_gemm_scratch(a_fp8, a_scale, w_fp8, w_scale, out=None):
    """The FP8 GEMM with split-K partial sums in the library's static device
    scratch (w8a8_block_gemm_scratch): no workspace argument, no allocation
    in the call.  Pass `out` to allocate nothing here either."""
    M, K = a_fp8.shape
    N = w_fp8.shape[0]
    _operand(a_fp8, torch.uint8, (M, K), "a_fp8")
    _operand(w_fp8, torch.uint8, (N, K), "w_fp8")
    _operand(a_scale, torch.float32, (M, _cdiv(K, 128)), "a_scale")
    _operand(w_scale, torch.float32, (_cdiv(N, 128), _cdiv(K, 128)), "w_scale")
    c = _out(out, torch.bfloat16, (M, N), a_fp8, "out")
    _check("w8a8_block_gemm_scratch",
           load().w8a8_block_gemm_scratch(_ptr(a_fp8), _ptr(a_scale), _ptr(w_fp8),
                                          _ptr(w_scale), M, N, K, _ptr(c), _stream(a_fp8)))
    return c


def _weight_multi(name, ws, outs, code_dtype, scale_shape):
    if len(ws) > MAX_WEIGHT_JOBS:
        raise ValueError(f"{name}: at most {MAX_WEIGHT_JOBS} weights per call")
    ws = [_bf16_bits(w, f"weights[{i}]") for i, w in enumerate(ws)]
    if outs is None:
        outs = [(None, None)] * len(ws)
    if len(outs) != len(ws):
        raise ValueError(f"{name}: one (codes, scales) pair per weight")
    res, jobs = [], (WeightJob * max(1, len(ws)))()
    for i, (w, (q, s)) in enumerate(zip(ws, outs)):
        N, K = w.shape
        q = _out(q, code_dtype, (N, K), w, f"outs[{i}][0]")
        s = _out(s, torch.float32, scale_shape(N, K), w, f"outs[{i}][1]")
        jobs[i] = WeightJob(_ptr(w), N, K, _ptr(q), _ptr(s))
        res.append((q, s))
    stream = _stream(ws[0]) if ws else torch.cuda.current_stream().cuda_stream
    _check(name, getattr(load(), name)(ctypes.addressof(jobs), len(ws), stream))
    return res


def fp8_weight_block_quant_multi(weights, outs=None):
    """Several Wt [N, K] bf16 weights in one launch -> [(codes uint8 [N, K],
    scales fp32 [ceil(N/128), ceil(K/128)])] (fp8_weight_block_quant_multi)."""
    return _weight_multi("fp8_weight_block_quant_multi", weights, outs, torch.uint8,
                         lambda N, K: (_cdiv(N, 128), _cdiv(K, 128)))


def int8_weight_channel_quant_multi(weights, outs=None):
    """Several Wt [N, K] bf16 weights in one launch -> [(codes int8 [N, K],
    scales fp32 [N])] (int8_weight_channel_quant_multi)."""
    return _weight_multi("int8_weight_channel_quant_multi", weights, outs, torch.int8,
                         lambda N, K: (N,))


def int8_weight_channel_quant(w: torch.Tensor, out=None, scale=None):
    """Wt [N, K] bf16 -> (codes int8 [N, K], scales fp32 [N])."""
    w = _bf16_bits(w, "w")
    N, K = w.shape
    q = _out(out, torch.int8, (N, K), w, "out")
    s = _out(scale, torch.float32, (N,), w, "scale")
    _check("int8_weight_channel_quant",
           load().int8_weight_channel_quant(_ptr(w), N, K, _ptr(q), _ptr(s), _stream(w)))
    return q, s


def int8_act_token_quant(a: torch.Tensor, out=None, scale=None):
    """A [M, K] bf16 -> (codes int8 [M, K], scales fp32 [M])."""
    a = _bf16_bits(a, "a")
    M, K = a.shape
    q = _out(out, torch.int8, (M, K), a, "out")
    s = _out(scale, torch.float32, (M,), a, "scale")
    _check("int8_act_token_quant",
           load().int8_act_token_quant(_ptr(a), M, K, _ptr(q), _ptr(s), _stream(a)))
    return q, s


def w8a8_int8_channel_gemm(a_i8, a_scale, w_i8, w_scale, out=None, workspace="auto"):
    """INT8 codes + per-row / per-channel scales -> C [M, N] bf16 (workspace
    as w8a8_block_gemm)."""
    M, K = a_i8.shape
    N = w_i8.shape[0]
    _operand(a_i8, torch.int8, (M, K), "a_i8")
    _operand(w_i8, torch.int8, (N, K), "w_i8")
    _operand(a_scale, torch.float32, (M,), "a_scale")
    _operand(w_scale, torch.float32, (N,), "w_scale")
    c = _out(out, torch.bfloat16, (M, N), a_i8, "out")
    ws = _workspace(workspace, M, N, K, a_i8)
    if ws is None:
        _check("w8a8_int8_channel_gemm",
               load().w8a8_int8_channel_gemm(_ptr(a_i8), _ptr(a_scale), _ptr(w_i8),
                                             _ptr(w_scale), M, N, K, _ptr(c), _stream(a_i8)))
    else:
        _check("w8a8_int8_channel_gemm_ws",
               load().w8a8_int8_channel_gemm_ws(_ptr(a_i8), _ptr(a_scale), _ptr(w_i8),
                                                _ptr(w_scale), M, N, K, _ptr(c), _ptr(ws),
                                                ws.numel(), _stream(a_i8)))
    return c


def fp8_kv_scale_recalibrate(x: torch.Tensor, out=None):
    """x [T, C] bf16 (a calibration batch of K, V or Q) -> scale fp32 [1]
    (stays on the device: fl32(max |x| / 448))."""
    x = _bf16_bits(x, "x")
    T, C = x.shape
    s = _out(out, torch.float32, (1,), x, "out")
    _check("fp8_kv_scale_recalibrate",
           load().fp8_kv_scale_recalibrate(_ptr(x), T, C, s.data_ptr(), _stream(x)))
    return s


def fp8_kv_cache_write(kv: torch.Tensor, slot_mapping: torch.Tensor, scale: torch.Tensor,
                       cache: torch.Tensor):
    """Quantize kv [T, C] bf16 with scale (fp32 [1], on the device) into rows
    slot_mapping[t] (int64 [T]; out-of-range / negative: skipped) of cache
    (uint8 [num_slots, C], updated in place).  Returns cache."""
    kv = _bf16_bits(kv, "kv")
    T, C = kv.shape
    _operand(slot_mapping, torch.int64, (T,), "slot_mapping")
    _operand(scale, torch.float32, (1,), "scale")
    if cache.dtype != torch.uint8 or cache.dim() != 2 or cache.shape[1] != C \
            or not cache.is_cuda or not cache.is_contiguous():
        raise ValueError(f"cache: expected a contiguous CUDA uint8 tensor [num_slots, {C}]")
    _check("fp8_kv_cache_write",
           load().fp8_kv_cache_write(_ptr(kv), _ptr(slot_mapping), T, C, scale.data_ptr(),
                                     _ptr(cache), cache.shape[0], _stream(kv)))
    return cache


def w8a8_block_gemm_grouped(aq: torch.Tensor, sa: torch.Tensor, wq: torch.Tensor,
                            sw: torch.Tensor, offsets: torch.Tensor, max_rows_per_expert: int,
                            out=None):
    """Rows of aq [M, K] (uint8, sorted by expert) x experts' wq [E, N, K]
    (uint8) with sa [M, K/128], sw [E, ceil(N/128), K/128] and
    offsets int64 [E + 1] (device) -> C bf16 [M, N]."""
    M, K = aq.shape
    E, N = wq.shape[0], wq.shape[1]
    _operand(aq, torch.uint8, (M, K), "aq")
    _operand(sa, torch.float32, (M, _cdiv(K, 128)), "sa")
    _operand(wq, torch.uint8, (E, N, K), "wq")
    _operand(sw, torch.float32, (E, _cdiv(N, 128), _cdiv(K, 128)), "sw")
    _operand(offsets, torch.int64, (E + 1,), "offsets")
    c = _out(out, torch.bfloat16, (M, N), aq, "out")
    _check("w8a8_block_gemm_grouped",
           load().w8a8_block_gemm_grouped(_ptr(aq), _ptr(sa), _ptr(wq), _ptr(sw), _ptr(offsets),
                                          E, M, N, K, int(max_rows_per_expert), _ptr(c),
                                          _stream(aq)))
    return c


def tis_token_weights(lp_train: torch.Tensor, lp_rollout: torch.Tensor, mask: torch.Tensor,
                      cap: float, mode: int = IS_TRUNCATE, out=None, row_stats=None, totals=None,
                      stats: bool = True):
    """Token-level importance weights of a batch: lp_train, lp_rollout fp32
    [B, T] (log-probabilities of the sampled tokens), mask uint8 [B, T]
    (nonzero = response token), truncation constant cap, mode IS_TRUNCATE
    (TIS) or IS_MASK (MIS).  Returns (weights fp32 [B, T], row_stats fp32
    [B, 4] or None, totals fp64 [4] or None)."""
    if lp_train.dim() != 2:
        raise ValueError("lp_train: expected [B, T]")
    B, T = lp_train.shape
    _operand(lp_train, torch.float32, (B, T), "lp_train")
    _operand(lp_rollout, torch.float32, (B, T), "lp_rollout")
    _operand(mask, torch.uint8, (B, T), "mask")
    w = _out(out, torch.float32, (B, T), lp_train, "out")
    rs = _out(row_stats, torch.float32, (B, 4), lp_train, "row_stats") if stats else None
    tt = _out(totals, torch.float64, (4,), lp_train, "totals") if stats else None
    _check("tis_token_weights",
           load().tis_token_weights(_ptr(lp_train), _ptr(lp_rollout), _ptr(mask), B, T,
                                    float(cap), int(mode), _ptr(w), _ptr(rs), _ptr(tt),
                                    _stream(lp_train)))
    return w, rs, tt


def attention_workspace_bytes(B: int, Hq: int, Hkv: int, D: int) -> int:
    """Workspace (bytes) fp8_kv_decode_attention_ws uses for these dimensions
    on the current device; 0 when the one-pass kernel is used."""
    key = ("att", torch.cuda.current_device(), int(B), int(Hq), int(Hkv), int(D))
    if key not in _ws_sizes:
        n = ctypes.c_int64(0)
        _check("fp8_kv_decode_attention_workspace_size",
               load().fp8_kv_decode_attention_workspace_size(int(B), int(Hq), int(Hkv), int(D),
                                                             ctypes.addressof(n)))
        _ws_sizes[key] = int(n.value)
    return _ws_sizes[key]


KV_RECAL_WORKSPACE_BYTES = 8192   # PRR_KV_RECAL_WORKSPACE_BYTES


def fp8_kv_cache_write_recalibrate(kv: torch.Tensor, slot_mapping: torch.Tensor,
                                   scale: torch.Tensor, cache: torch.Tensor, new_scale=None,
                                   workspace=None):
    """One pass over kv [T, C] bf16: fp8_kv_cache_write(kv, slot_mapping,
    scale, cache), and the next step's scale fl32(max |kv| / 448) into
    new_scale (fp32 [1] on the device; may be `scale` itself, updated in
    place).  workspace: a uint8 CUDA tensor of at least
    KV_RECAL_WORKSPACE_BYTES, or None for a new one.  Returns new_scale."""
    kv = _bf16_bits(kv, "kv")
    T, C = kv.shape
    _operand(slot_mapping, torch.int64, (T,), "slot_mapping")
    _operand(scale, torch.float32, (1,), "scale")
    if cache.dtype != torch.uint8 or cache.dim() != 2 or cache.shape[1] != C \
            or not cache.is_cuda or not cache.is_contiguous():
        raise ValueError(f"cache: expected a contiguous CUDA uint8 tensor [num_slots, {C}]")
    ns = _out(new_scale, torch.float32, (1,), kv, "new_scale")
    if workspace is None:
        workspace = torch.empty((KV_RECAL_WORKSPACE_BYTES,), dtype=torch.uint8, device=kv.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace: expected a contiguous CUDA uint8 tensor")
    _check("fp8_kv_cache_write_recalibrate",
           load().fp8_kv_cache_write_recalibrate(_ptr(kv), _ptr(slot_mapping), T, C,
                                                 scale.data_ptr(), _ptr(cache), cache.shape[0],
                                                 ns.data_ptr(), _ptr(workspace),
                                                 workspace.numel(), _stream(kv)))
    return ns


def fp8_kv_cache_write_recalibrate_multi(kvs, slot_mapping: torch.Tensor, scales, caches,
                                         new_scales=None, workspace=None):
    """fp8_kv_cache_write_recalibrate for several tensors sharing the slot
    mapping (K and V of a step), in one launch over their rows: kvs, scales,
    caches and new_scales are sequences of the single call's arguments
    (new_scales[i] may be scales[i]; None: new tensors).  workspace: a uint8
    CUDA tensor of at least len(kvs) x KV_RECAL_WORKSPACE_BYTES, or None for
    a new one.  Returns the new scales."""
    n = len(kvs)
    if not (len(scales) == len(caches) == n) or n > MAX_KV_JOBS:
        raise ValueError(f"kvs, scales, caches: {n} each, at most {MAX_KV_JOBS}")
    if n == 0:
        return []
    kvs = [_bf16_bits(k, "kv") for k in kvs]
    T, C = kvs[0].shape
    if any(k.shape != (T, C) for k in kvs):
        raise ValueError("kvs: every tensor [T, C] alike")
    _operand(slot_mapping, torch.int64, (T,), "slot_mapping")
    num_slots = caches[0].shape[0] if caches[0].dim() == 2 else -1
    for sc, ca in zip(scales, caches):
        _operand(sc, torch.float32, (1,), "scale")
        if ca.dtype != torch.uint8 or ca.dim() != 2 or tuple(ca.shape) != (num_slots, C) \
                or not ca.is_cuda or not ca.is_contiguous():
            raise ValueError(f"caches: contiguous CUDA uint8 tensors [num_slots, {C}], all alike")
    if new_scales is None:
        new_scales = [None] * n
    ns = [_out(x, torch.float32, (1,), kvs[0], "new_scale") for x in new_scales]
    need = n * KV_RECAL_WORKSPACE_BYTES
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=kvs[0].device)
    elif workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace: expected a contiguous CUDA uint8 tensor")
    jobs = (KvJob * n)(*[KvJob(_ptr(k), sc.data_ptr(), _ptr(ca), x.data_ptr())
                         for k, sc, ca, x in zip(kvs, scales, caches, ns)])
    _check("fp8_kv_cache_write_recalibrate_multi",
           load().fp8_kv_cache_write_recalibrate_multi(ctypes.addressof(jobs), n,
                                                       _ptr(slot_mapping), T, C, num_slots,
                                                       _ptr(workspace), workspace.numel(),
                                                       _stream(kvs[0])))
    return ns


def fp8_kv_decode_attention(q: torch.Tensor, q_scale: torch.Tensor, k_cache: torch.Tensor,
                            v_cache: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                            block_table: torch.Tensor, seq_lens: torch.Tensor, Hkv: int,
                            page: int, softmax_scale: float | None = None, out=None,
                            workspace="auto"):
    """Decode attention over the FP8 KV cache: q bf16 [B, Hq, D]; scales fp32
    [1] on the device; caches uint8 [num_slots, Hkv * D]; block_table int32
    [B, max_blocks]; seq_lens int32 [B].  Returns bf16 [B, Hq, D].  With a
    workspace (by default one of the size the library asks for) the batch's
    tokens are split evenly over the CUs (fp8_kv_decode_attention_ws);
    workspace=None runs the one-pass kernel."""
    if q.dim() != 3:
        raise ValueError("q: expected [B, Hq, D]")
    B, Hq, D = q.shape
    if q.dtype not in (torch.bfloat16, torch.int16) or not q.is_cuda or not q.is_contiguous():
        raise ValueError("q: expected a contiguous CUDA bf16 tensor")
    for t, name in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        _operand(t, torch.float32, (1,), name)
    num_slots = k_cache.shape[0]
    _operand(k_cache, torch.uint8, (num_slots, Hkv * D), "k_cache")
    _operand(v_cache, torch.uint8, (num_slots, Hkv * D), "v_cache")
    if block_table.dim() != 2:
        raise ValueError("block_table: expected [B, max_blocks]")
    _operand(block_table, torch.int32, (B, block_table.shape[1]), "block_table")
    _operand(seq_lens, torch.int32, (B,), "seq_lens")
    o = _out(out, torch.bfloat16, (B, Hq, D), q, "out")
    c = float(1.0 / D ** 0.5) if softmax_scale is None else float(softmax_scale)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace: 'auto', None or a uint8 CUDA tensor")
        n = attention_workspace_bytes(B, Hq, Hkv, D) if B > 0 and Hq > 0 and Hkv > 0 else 0
        workspace = torch.empty((n,), dtype=torch.uint8, device=q.device) if n else None
    elif workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_cuda
                                    or not workspace.is_contiguous()):
        raise ValueError("workspace: expected a contiguous CUDA uint8 tensor")
    args = (_ptr(q), q_scale.data_ptr(), _ptr(k_cache), _ptr(v_cache), k_scale.data_ptr(),
            v_scale.data_ptr(), _ptr(block_table), _ptr(seq_lens), B, Hq, Hkv, D, page,
            block_table.shape[1], num_slots, c, _ptr(o))
    if workspace is None:
        _check("fp8_kv_decode_attention", load().fp8_kv_decode_attention(*args, _stream(q)))
    else:
        _check("fp8_kv_decode_attention_ws",
               load().fp8_kv_decode_attention_ws(*args, _ptr(workspace), workspace.numel(),
                                                 _stream(q)))
    return o
