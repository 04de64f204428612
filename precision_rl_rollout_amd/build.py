"""Build libprr.so (HIP for gfx950) in-tree with hipcc.

``python -m precision_rl_rollout_amd.build`` compiles every source under
``csrc/`` into ``precision_rl_rollout_amd/libprr.so``.  No GPU is needed:
hipcc cross-compiles for gfx950.  Sources compile in parallel to objects
under ``_build/`` (git-ignored), which are then linked.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libprr.so")
OBJ_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "quant_fp8.hip", "quant_int8.hip", "gemm.hip", "gemm_decode.hip",
           "gemm_prefill.hip", "kv_fp8.hip", "tis.hip", "attention.hip"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
# No fast-math or denormal-flush flags: the quantizers rely on IEEE fp32
# division with subnormals kept.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _filter(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)


def _compile(src: str) -> tuple[str, int, str]:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    return obj, res.returncode, _filter(res.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    jobs = max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, srcs))
    for (obj, rc, err), src in zip(results, srcs):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({rc}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *[r[0] for r in results],
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{_filter(res.stderr)}")
    os.replace(tmp, LIB)
    return LIB


def asan_runtime() -> str | None:
    """The compiler's shared AddressSanitizer runtime (to preload into a
    process that loads the instrumented library), or None."""
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def build_asan_abi() -> str:
    """A copy of the library whose host-side ABI layer (api.cpp: argument,
    pointer and device checks) is built with AddressSanitizer; the kernels'
    objects are the regular ones (the sanitizer applies to host code only).
    Returns the path of _build/libprr_asan.so; it loads only into a process
    that preloads asan_runtime()."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    others = [s for s in SOURCES if s != "api.cpp"]
    objs = [os.path.join(OBJ_DIR, s + ".o") for s in others]
    missing = [os.path.join(CSRC, s) for s, o in zip(others, objs) if not os.path.exists(o)]
    if missing:
        with ThreadPoolExecutor(max(1, min(len(missing), os.cpu_count() or 1, 16))) as ex:
            for obj, rc, err in ex.map(_compile, missing):
                if rc != 0:
                    raise RuntimeError(f"hipcc failed on {obj}:\n{err}")
    api_obj = os.path.join(OBJ_DIR, "api_asan.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           "-shared-libsan"]
    cmd = [hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san,
           "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc (asan) failed:\n{_filter(res.stderr)}")
    lib = os.path.join(OBJ_DIR, "libprr_asan.so")
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *san, api_obj, *objs,
           "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link (asan) failed:\n{_filter(res.stderr)}")
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
