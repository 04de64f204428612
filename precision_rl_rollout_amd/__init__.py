"""MI355X-native 8-bit rollout kernels: FP8 e4m3 block re-quantization, W8A8
block-scaled GEMM with bf16 output, and the INT8 per-channel variant.

The compute lives in ``libprr.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/prr.h``).  ``precision_rl_rollout_amd.binding`` is the
thin ctypes layer over it; importing this package loads nothing, so the
input generators in ``precision_rl_rollout_amd.workloads`` can be used on a
machine without a GPU.
"""

__all__ = ["binding", "workloads", "build"]
