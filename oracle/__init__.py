"""CPU oracle for the 8-bit rollout hot path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP kernels in
``libprr.so`` and their Python binding) never imports, links or calls it,
and this package imports nothing from the product path.

What it computes, with the passage each part follows:

* ``oracle.e4m3`` -- the OCP FP8 E4M3 code (bias 7, no infinities, one NaN
  mantissa pattern, largest finite 448): saturating round-to-nearest-even
  encode by explicit bit construction, and the closed-form decode.  The
  pages name FP8 without a sub-format; e4m3 with a 448 limit is the format
  the blockwise FP8 rollout stack of "FP8-RL: A Practical and Stable
  Low-Precision Stack for LLM Reinforcement Learning" (abstract, item (i))
  is read to use.
* ``oracle.quant`` -- per-step re-quantization of bf16 weights (128 x 128
  blocks) and activations (1 x 128 per-token groups) into e4m3 with one fp32
  scale ``amax / 448`` per block (FP8-RL abstract: policy weights change
  every step, so they are quantized again every step; item (i): blockwise
  FP8 W8A8 linear layers), and the INT8 variant with per-output-channel
  weight scales and per-token activation scales ``amax / 127`` (FlashRL
  article, sections on 8-bit rollout and online quantization with parameter
  updates: INT8 and FP8 rollout).
* ``oracle.kv`` -- the FP8 KV cache: one scale ``amax / 448`` per tensor,
  recalibrated every step, and quantize-on-write of token rows into cache
  slots (FP8-RL abstract, item (ii): FP8 KV cache with per-step QKV scale
  recalibration; granularity and write rule are readings, listed there).
* ``oracle.attention`` -- decode attention over the FP8 KV cache: the
  query quantized with its own per-tensor scale, scores and softmax in fp64
  over the paged cache's codes, the output rounded once to bf16 (FP8-RL
  abstract, item (ii): FP8 KV cache with per-step Q/K/V scales; the
  attention details are readings, listed there).
* ``oracle.gemm`` -- also the mixture-of-experts grouping of the FP8 layer:
  token rows sorted by expert, each group multiplied by its expert's weight
  (FP8-RL abstract: dense and MoE models).
* ``oracle.tis`` -- token-level importance weights for rollout correction:
  the trainer-to-rollout probability ratio of each sampled token, truncated
  (TIS) or masked (MIS) at a constant, with per-sequence statistics
  (FP8-RL abstract, item (iii); FlashRL article, section on the
  rollout-training mismatch; formula and constant are readings, listed
  there).
* ``oracle.gemm`` -- the W8A8 linear layer: fp64 accumulation over the
  exactly decoded 8-bit operands with the per-K-block (FP8) or per-row and
  per-channel (INT8) scales, rounded once to bf16.

Precision: the scale ``fl32(amax / 448)`` and the quotient ``fl32(x / s)``
are IEEE binary32 operations, correctly rounded, with subnormals honoured;
everything else is exact integer arithmetic or fp64.  numpy's float32
division is the host's correctly rounded ``divss``; the import-time check
below refuses to run if the process flushes subnormals.

Parity pins live in ``tests/test_oracle_*.py`` (closed forms, brute force,
library cross-checks, exact rational arithmetic, invariants).
"""

import numpy as _np


def _check_subnormals() -> None:
    tiny = _np.float32(2.0 ** -149)
    with _np.errstate(all="ignore"):
        half_min_normal = _np.float32(2.0 ** -126) / _np.float32(2.0)
    if tiny == 0 or half_min_normal == 0:
        raise RuntimeError("oracle: this process flushes float32 subnormals "
                           "to zero; the oracle's fp32 steps would be wrong")


_check_subnormals()

from . import e4m3, quant, gemm  # noqa: E402,F401
