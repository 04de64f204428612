"""MI355X-native 8-bit rollout kernels: FP8 e4m3 block re-quantization (of
whole weights or of shards as they arrive), W8A8 block-scaled GEMM with bf16
output (dense and grouped over experts), the INT8 per-channel variant, the
FP8 KV cache (scale recalibration, quantize-on-write, decode attention) and
token-level TIS / MIS importance weights.

The compute lives in ``libprr.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/prr.h``).  ``precision_rl_rollout_amd.binding`` is the
thin ctypes layer over it; importing this package loads nothing, so the
input generators in ``precision_rl_rollout_amd.workloads`` can be used on a
machine without a GPU.
"""

__all__ = ["binding", "workloads", "build"]
