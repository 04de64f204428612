"""bench.py's command line on a machine without a GPU (CPU): it refuses more
than one GPU with a message, refuses to run without a GPU, and its work
counts match the formulas it documents."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in r.stderr


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="a GPU is present")
def test_no_gpu_is_reported():
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0 and "needs a GPU" in r.stderr


def test_work_counts():
    # bf16 read + code written + one fp32 scale per block
    assert bench.quant_bytes(37888, 3584, 296 * 28) == 3 * 37888 * 3584 + 4 * 296 * 28
    # weight codes + activation codes + scales + bf16 output
    M, N, K = 64, 37888, 3584
    assert bench.gemm_bytes(M, N, K, M * 28, 296 * 28) == N * K + M * K + 4 * (M * 28 + 296 * 28) + 2 * M * N
    assert bench.cdiv(37888, 128) == 296 and bench.cdiv(1, 128) == 1
