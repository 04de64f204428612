"""Per-step re-quantization of bf16 weights and activations (CPU oracle).

FP8 (FP8-RL, abstract: policy weights change every step and are quantized
again every step; item (i): blockwise FP8 W8A8 linear layers):

* weights ``Wt [N, K]`` in 128 x 128 blocks, activations ``A [M, K]`` in
  1 x 128 groups along K (one token, 128 consecutive input features);
* per block: ``amax = max |x|`` over the block's valid elements (partial
  edge blocks use what is there), ``s = fl32(amax / 448)``;
* per element: ``q = E4M3_sat_RNE(fl32(x / s))``; an all-zero block has
  ``s = 0`` and its codes are the signed zeros of its inputs.

INT8 (FlashRL article, INT8 rollout and online quantization with parameter
updates; the granularity is not stated there and is read as symmetric
per-output-channel for weights and per-token over the whole K for
activations):

* per row: ``s = fl32(amax / 127)``, ``q = clamp(RNE(fl32(x / s)), -127, 127)``;
  an all-zero row has ``s = 0`` and codes 0.

``fl32(.)`` is an IEEE binary32 operation, correctly rounded.
"""

from __future__ import annotations

import numpy as np

from . import e4m3

BLOCK = 128
FP8_DIV = np.float32(448.0)
INT8_DIV = np.float32(127.0)


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact: the bits become the top
    half of the float32 word)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _check_finite(x: np.ndarray) -> None:
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle: non-finite input (the method is defined "
                         "for finite bf16 values only)")


def _quotient(x: np.ndarray, s: np.float32) -> np.ndarray:
    """fl32(x / s); for s == 0 every x in the block is a signed zero and the
    quotient is taken to be x itself."""
    if s == 0:
        return x.astype(np.float32)
    with np.errstate(under="ignore"):
        return (x / s).astype(np.float32)


def fp8_block_scale(x_block: np.ndarray) -> np.float32:
    """s = fl32(max|x| / 448) of one block of float32 values."""
    amax = np.float32(np.max(np.abs(x_block)))
    with np.errstate(under="ignore"):
        return np.float32(amax / FP8_DIV)


def _block_amax(x: np.ndarray, rb: int, cb: int) -> np.ndarray:
    """max |x| over each rb x cb block (partial edge blocks: their valid
    elements; zero padding cannot raise a maximum of magnitudes)."""
    R, C = x.shape
    nr, nc = -(-R // rb), -(-C // cb)
    pad = np.zeros((nr * rb, nc * cb), dtype=np.float32)
    pad[:R, :C] = np.abs(x)
    return pad.reshape(nr, rb, nc, cb).max(axis=(1, 3))


def _divide_and_encode(x: np.ndarray, s_full: np.ndarray, encode) -> np.ndarray:
    """encode(fl32(x / s)) elementwise, with x itself where s == 0; done in
    row chunks to bound the temporaries."""
    out = np.empty(x.shape, dtype=np.uint8 if encode is e4m3.encode else np.int8)
    step = max(1, (1 << 22) // max(1, x.shape[1]))
    for r in range(0, x.shape[0], step):
        xs, ss = x[r:r + step], s_full[r:r + step]
        with np.errstate(divide="ignore", invalid="ignore", under="ignore"):
            v = np.where(ss == 0, xs, xs / np.where(ss == 0, np.float32(1), ss))
        out[r:r + step] = encode(v.astype(np.float32))
    return out


def fp8_weight_block_quant(w_bits) -> tuple[np.ndarray, np.ndarray]:
    """Wt bf16 [N, K] -> (codes uint8 [N, K], scales float32 [ceil(N/128),
    ceil(K/128)])."""
    x = bf16_to_f32(w_bits)
    _check_finite(x)
    N, K = x.shape
    amax = _block_amax(x, BLOCK, BLOCK)
    with np.errstate(under="ignore"):
        scales = (amax / FP8_DIV).astype(np.float32)
    s_full = np.repeat(np.repeat(scales, BLOCK, axis=0)[:N], BLOCK, axis=1)[:, :K]
    return _divide_and_encode(x, s_full, e4m3.encode), scales


def fp8_weight_blocks(w_bits, block_ids) -> list[tuple[np.ndarray, np.float32]]:
    """The same as ``fp8_weight_block_quant`` for selected blocks only:
    returns [(codes of block (i, j), scale of block (i, j))]."""
    out = []
    for i, j in block_ids:
        blk = bf16_to_f32(w_bits[i * BLOCK:(i + 1) * BLOCK,
                                 j * BLOCK:(j + 1) * BLOCK])
        _check_finite(blk)
        s = fp8_block_scale(blk)
        out.append((e4m3.encode(_quotient(blk, s)), s))
    return out


def fp8_act_token_quant(a_bits) -> tuple[np.ndarray, np.ndarray]:
    """A bf16 [M, K] -> (codes uint8 [M, K], scales float32 [M, ceil(K/128)])."""
    x = bf16_to_f32(a_bits)
    _check_finite(x)
    M, K = x.shape
    amax = _block_amax(x, 1, BLOCK)
    with np.errstate(under="ignore"):
        scales = (amax / FP8_DIV).astype(np.float32)
    s_full = np.repeat(scales, BLOCK, axis=1)[:, :K]
    return _divide_and_encode(x, s_full, e4m3.encode), scales


def int8_encode(v: np.ndarray) -> np.ndarray:
    """clamp(RNE(v), -127, 127) as int8 (np.rint rounds half to even)."""
    return np.clip(np.rint(v.astype(np.float64)), -127, 127).astype(np.int8)


def _int8_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    with np.errstate(under="ignore"):
        scales = (amax.astype(np.float32) / INT8_DIV).astype(np.float32)
    codes = _divide_and_encode(x, np.repeat(scales[:, None], x.shape[1], axis=1), int8_encode)
    codes[scales == 0] = 0
    return codes, scales


def int8_weight_channel_quant(w_bits) -> tuple[np.ndarray, np.ndarray]:
    """Wt bf16 [N, K] -> (codes int8 [N, K], scales float32 [N])."""
    x = bf16_to_f32(w_bits)
    _check_finite(x)
    return _int8_rows(x)


def int8_act_token_quant(a_bits) -> tuple[np.ndarray, np.ndarray]:
    """A bf16 [M, K] -> (codes int8 [M, K], scales float32 [M])."""
    x = bf16_to_f32(a_bits)
    _check_finite(x)
    return _int8_rows(x)
