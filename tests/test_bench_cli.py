"""bench.py's command line on a machine without a GPU (CPU): it refuses more
than one GPU with a message, refuses to run without a GPU, its work counts
match the formulas it documents, and its HBM traffic figures come only from
counter records taken on the kernels' current sources."""

import glob
import json
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


def _profile(root, workload, table):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", f"{workload}_hbm_traffic.md"), "w") as f:
        f.write("# counters\n\n```json\n" + json.dumps(table) + "\n```\n")


def test_measured_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    """A traffic record counts only while the kernel's sources are the ones
    it was taken on (their digest); a changed source, a missing record or a
    missing profile give None."""
    csrc = tmp_path / "precision_rl_rollout_amd" / "csrc"
    csrc.mkdir(parents=True)
    files = bench.KERNEL_SOURCES["w8a8_block_gemm@decode7b_upgate"]
    for n in files:
        (csrc / n).write_text(f"// {n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w8a8_block_gemm", "decode7b_upgate") is None   # no profile
    digest = bench._sources_digest(files)
    _profile(str(tmp_path), "decode7b_upgate",
             {"w8a8_block_gemm@decode7b_upgate": {"bytes_per_launch": 123, "sources": digest}})
    assert bench.measured_traffic("w8a8_block_gemm", "decode7b_upgate") == 123
    assert bench.measured_traffic("w8a8_int8_channel_gemm", "decode7b_upgate") is None
    (csrc / files[0]).write_text("// edited\n")
    assert bench.measured_traffic("w8a8_block_gemm", "decode7b_upgate") is None


def test_committed_traffic_records_name_known_kernels():
    """Every record in the committed counter summaries is keyed
    kernel@workload, for a kernel whose sources bench.py knows, with a
    positive byte count and a 16-digit source digest."""
    paths = glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.md"))
    assert paths
    for path in paths:
        text = open(path).read()
        table = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        workload = os.path.basename(path)[: -len("_hbm_traffic.md")]
        for key, rec in table.items():
            kernel, _, wl = key.partition("@")
            assert wl == workload, (path, key)
            assert key in bench.KERNEL_SOURCES or kernel in bench.KERNEL_SOURCES, (path, key)
            assert rec["bytes_per_launch"] > 0 and len(rec["sources"]) == 16, (path, key)
