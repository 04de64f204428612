"""FP8 KV cache: per-step scale recalibration and quantize-on-write (CPU
oracle).  TEST INFRASTRUCTURE ONLY (see the package header).

"FP8-RL: A Practical and Stable Low-Precision Stack for LLM Reinforcement
Learning", abstract, item (ii): FP8 is extended to the KV cache, with the
Q/K/V scales recalibrated at every step (the policy weights, and so the
projections that produce Q, K and V, change every step).  The pages give no
granularity, format or write rule; the readings taken here:

* one scale per tensor (per layer, separately for K, V and Q), recalibrated
  from a batch of that tensor: ``s = fl32(amax / 448)`` over all of its
  elements -- the same rule as a weight block, with the whole tensor as the
  block;
* quantize-on-write: a token row ``x`` (``C = kv_heads * head_dim`` bf16
  values) lands in cache row ``slot`` as ``E4M3_sat_RNE(fl32(x / s))``;
  values above the calibration range saturate to +-448, including values
  whose quotient ``x / s`` overflows binary32 (a stale scale far below the
  new values); ``s == 0`` writes the signed zeros of ``x`` (the
  all-zero-block rule);
* a slot outside ``[0, num_slots)`` (negative: a padding token) is skipped;
  distinct tokens map to distinct slots, and cache rows no token maps to are
  left as they were.
"""

from __future__ import annotations

import numpy as np

from . import e4m3
from .quant import FP8_DIV, _check_finite, _quotient, bf16_to_f32


def kv_scale(x_bits) -> np.float32:
    """bf16 [T, C] (any shape) -> s = fl32(max |x| / 448)."""
    x = bf16_to_f32(x_bits)
    _check_finite(x)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    with np.errstate(under="ignore"):
        return np.float32(amax / FP8_DIV)


def kv_encode_rows(x_bits, s: np.float32) -> np.ndarray:
    """bf16 [T, C] -> e4m3 codes [T, C] with the tensor scale s; s == 0
    gives the signed zeros of x (rows may be nonzero here, unlike an
    all-zero weight block, so this is spelled out)."""
    x = bf16_to_f32(x_bits)
    _check_finite(x)
    if np.float32(s) == 0:
        return np.where(np.signbit(x), np.uint8(0x80), np.uint8(0x00)).astype(np.uint8)
    with np.errstate(over="ignore"):
        v = _quotient(x, np.float32(s))
    # A scale from an earlier batch can be so small that fl32(x / s) leaves
    # the binary32 range: such a quotient is a value above the calibrated
    # range like any other and saturates to +-448 (the sign is that of x).
    v = np.where(np.isinf(v), np.copysign(np.float32(448.0), v), v).astype(np.float32)
    return e4m3.encode(v)


def kv_cache_write(cache: np.ndarray, x_bits, slot_mapping, s: np.float32) -> np.ndarray:
    """Returns a copy of ``cache`` (uint8 [num_slots, C]) with row
    ``slot_mapping[t]`` replaced by the codes of token row ``t`` for every
    token whose slot is in range."""
    out = np.array(cache, dtype=np.uint8, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    codes = kv_encode_rows(x_bits, s)
    keep = (slots >= 0) & (slots < out.shape[0])
    if len(np.unique(slots[keep])) != int(keep.sum()):
        raise ValueError("oracle: two tokens map to one cache slot")
    out[slots[keep]] = codes[keep]
    return out
