"""The host-side ABI checks under AddressSanitizer: tests/test_abi.py run in
a child process against a build of the library whose ABI layer (api.cpp) is
instrumented, with the sanitizer runtime preloaded.  Any invalid host
memory access in an argument check, status string or device query aborts
that child, which fails this test."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


@pytest.mark.skipif(_gpu_visible(), reason="host-only check; runs in a process without a GPU")
def test_abi_checks_under_host_address_sanitizer():
    from precision_rl_rollout_amd import build
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    lib = build.build_asan_abi()
    env = dict(os.environ, LD_PRELOAD=rt, PRR_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    probe = ("import ctypes; ctypes.CDLL(None).__asan_init; "
             "from precision_rl_rollout_amd import binding; "
             "assert binding.LIB_PATH == %r; binding.load(); print('asan-active')" % lib)
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0 and "asan-active" in r.stdout, r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_abi.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])
    assert "passed" in r.stdout
