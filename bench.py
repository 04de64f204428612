"""Benchmark of the 8-bit rollout hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The default workload is the 7B-class decode FFN up/gate layer (A [64,
3584], Wt [37888, 3584]).  One step is one decode pass of it: FP8
per-token-group quantization of the activations and the W8A8 block-scaled
GEMM against the FP8 weight (quantized before; five copies alternate so
that no step finds the weight in the 256 MB last-level cache).  Inputs are
synthetic (seeded, see precision_rl_rollout_amd.workloads) and resident in
HBM before the timed region.

Prints one JSON line.  ``value`` and ``roofline`` are the GEMM's own
algorithmic GB/s (HIP events on the launch stream around its calls in the
timed steps) against the 8 TB/s HBM peak; ``prefill`` carries the other
half of the metric, the FP8 GEMM of the 32B-class prefill up/gate layer
(M 8192, N 27648, K 5120) in TFLOP/s against the 5.0 PFLOP/s FP8 peak;
``requant_step`` is the whole per-step path at the decode shape (FP8 and
INT8 weight re-quantization, activation quantization and GEMM) with every
kernel's duration; ``cpu_baseline`` (and ``prefill.cpu_baseline``) time
the CPU oracle on the same GEMM (a row sample of the prefill one).

Other workloads (``--workload``): ``decode32b_sweep`` (GEMMs at M = 1..128,
N 27648, K 5120, cold weights), ``prefill32b`` (M 8192 up/gate and down
GEMMs, TFLOP/s), ``stack32b_requant`` (FP8 and INT8 re-quantization of a
32B-class layer's seven weights), ``kv32b_prefill`` (FP8 KV-cache
quantize-on-write and scale recalibration of a 16,384-token prefill's K
and V in one call, beside the per-tensor and the separate calls),
``moe_decode`` (a 128-expert top-8 decode layer: weight re-quantization of
every expert, activation quantization, the grouped GEMM), ``tis_batch``
(TIS and MIS token weights of 1024 responses padded to 8192 tokens),
``stack32b_gemm`` (the decode GEMMs of a 32B layer stack at M = 1 and 64),
``att32b_decode`` (decode attention over an FP8 KV cache: 64 sequences of
1024-8192 tokens, 40 query heads over 8 KV heads; the call with its
workspace, which splits the batch's tokens over the CUs; ``batch_sizes``
adds the first 1, 2, 8 and 64 sequences with and without the split),
``sync32b_requant`` (quantize-on-receive: the 32B up/gate weight arriving
in 8 shards from pinned host memory, each quantized into place in the full
FP8 weight while the next is in transfer).  Steps of these workloads run
behind a short hold of the launch stream, so that the host has queued
them before the GPU starts (several of their kernels are shorter than a
Python call into the binding); their time is the GPU time of the queued
steps, and ``timing`` notes the host's own time per step beside it.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W8A8 block GEMM TFLOP/s (% FP8 peak); decode-shape HBM GB/s (% peak)"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
INT8_PEAK_TOPS = 5000.0


# ---------------------------------------------------------------- work counts
def quant_bytes(rows, K, units):
    """bf16 read + code written + one fp32 scale per block / group / row."""
    return 3 * rows * K + 4 * units


def gemm_bytes(M, N, K, a_scales, w_scales):
    """FP8/INT8 weight + activation codes, their scales, bf16 output."""
    return N * K + M * K + 4 * (a_scales + w_scales) + 2 * M * N


def cdiv(a, b):
    return -(-a // b)


# ---------------------------------------------------------------- helpers
def _sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "precision_rl_rollout_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "fp8_weight_block_quant": ["quant_fp8.hip", "prr_device.h"],
    "fp8_weight_block_quant_multi": ["quant_fp8.hip", "prr_device.h"],
    "int8_weight_channel_quant_multi": ["quant_int8.hip", "prr_device.h"],
    "fp8_act_token_quant": ["quant_fp8.hip", "prr_device.h"],
    "int8_weight_channel_quant": ["quant_int8.hip", "prr_device.h"],
    "int8_act_token_quant": ["quant_int8.hip", "prr_device.h"],
    "w8a8_block_gemm": ["gemm.hip", "prr_device.h"],
    "w8a8_int8_channel_gemm": ["gemm.hip", "prr_device.h"],
    # M <= 64 runs the persistent decode kernel.
    "w8a8_block_gemm@decode7b_upgate": ["gemm_decode.hip", "mfma.h", "prr_device.h"],
    "w8a8_int8_channel_gemm@decode7b_upgate": ["gemm_decode.hip", "mfma.h", "prr_device.h"],
    "w8a8_block_gemm_grouped": ["gemm_decode.hip", "mfma.h", "prr_device.h"],
    "tis_token_weights": ["tis.hip", "prr_device.h"],
    "fp8_kv_scale_recalibrate": ["kv_fp8.hip", "prr_device.h"],
    "fp8_kv_cache_write": ["kv_fp8.hip", "prr_device.h"],
    "fp8_kv_cache_write_recalibrate": ["kv_fp8.hip", "prr_device.h"],
    "fp8_kv_cache_write_recalibrate_multi": ["kv_fp8.hip", "prr_device.h"],
    "fp8_kv_decode_attention": ["attention.hip", "prr_device.h"],
    # M = 8192 runs the many-token kernel.
    "w8a8_block_gemm@prefill32b": ["gemm_prefill.hip", "mfma.h", "prr_device.h"],
    "w8a8_int8_channel_gemm@prefill32b": ["gemm_prefill.hip", "mfma.h", "prr_device.h"],
}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if
    it was taken on the kernel's current sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if "```json" not in text:
        return None
    table = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    rec = table.get(f"{kernel}@{workload}")
    files = KERNEL_SOURCES.get(f"{kernel}@{workload}", KERNEL_SOURCES[kernel])
    if not rec or rec.get("sources") != _sources_digest(files):
        return None
    return rec.get("bytes_per_launch")


class Timer:
    """Per-call HIP event pairs on torch's current stream (the stream the
    binding launches on); with `only`, for calls of that name only."""

    def __init__(self, torch, only=None):
        self.torch = torch
        self.only = only
        self.pairs = {}

    def run(self, name, fn):
        if self.only is not None and name != self.only:
            return fn()
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        out = fn()
        e.record()
        self.pairs.setdefault(name, []).append((s, e))
        return out

    def avg_us(self):
        return {k: 1e3 * float(np.mean([s.elapsed_time(e) for s, e in v]))
                for k, v in self.pairs.items()}


# One note per timed_steps pass ({step, host_us_per_step, queued}); main()
# attaches them to the line as "timing".
TIMINGS = []


def hold_stream(torch, us, mark=None):
    """Keep the launch stream busy for about `us` microseconds with torch's
    one-thread spin kernel (bounded: it counts down a fixed number of
    clock cycles), so that the host queues the calls that follow ahead of
    the GPU.  Kernels of 10-20 us are shorter than a Python call into the
    binding: unheld, the GPU waits on the host between them and event pairs
    time the host's launch path, not the kernels.  The spin's cycles per
    microsecond follow the clock, so a short spin is timed first, at the
    clock of the moment.  `mark`, an event, is recorded just before the
    hold itself."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    torch.cuda._sleep(200_000)
    e1.record()
    torch.cuda.synchronize()
    per_us = 200_000 / max(1.0, e0.elapsed_time(e1) * 1e3)
    if mark is not None:
        mark.record()
    torch.cuda._sleep(int(us * per_us))


def timed_steps(torch, step, args):
    """Warm-up steps; a short instrumented pass (untimed) that gives every
    kernel's duration and names the dominant one; then the K timed steps,
    with HIP events around the dominant kernel's calls only.  (An event
    pair around every call leaves the GPU idle ~3.5 us per marker: the
    6-kernel decode step measured 258 us instrumented, 213 us without,
    and 213 us as a HIP graph replay.)  Both passes start behind a hold of
    the launch stream (hold_stream) four times as long as the host took to
    issue that many warm-up steps (the instrumented steps' event markers
    slow the host down), so the steps run back to back on the GPU; the step
    time is the GPU time of the K queued steps, between a HIP event after
    the hold and one after the last step (the host's own time per step is
    noted in TIMINGS, with whether the hold outlasted the host's issue of
    the K steps).  step(i, timer) runs step i.
    Returns (seconds per step, {kernel: us}, dominant kernel)."""
    t0 = time.perf_counter()
    for i in range(args.warmup):
        step(i, None)
    host_us = (time.perf_counter() - t0) * 1e6 / max(1, args.warmup)
    torch.cuda.synchronize()
    n_pre = max(1, min(args.steps, 10))
    hold_stream(torch, 4 * host_us * n_pre + 500)
    pre = Timer(torch)
    for i in range(n_pre):
        step(i, pre)
    torch.cuda.synchronize()
    us = pre.avg_us()
    dom = max(us, key=us.get)
    timer = Timer(torch, only=dom)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    hold_stream(torch, 4 * host_us * args.steps + 500, mark=ev[0])
    ev[1].record()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, timer)
    enqueue_us = (time.perf_counter() - t0) * 1e6
    ev[2].record()
    torch.cuda.synchronize()
    dt = ev[1].elapsed_time(ev[2]) * 1e-3 / args.steps
    us[dom] = timer.avg_us()[dom]
    hold_us = ev[0].elapsed_time(ev[1]) * 1e3
    TIMINGS.append({"step": getattr(step, "__name__", "step"), "steps": args.steps,
                    "gpu_us_per_step": round(dt * 1e6, 2),
                    "host_us_per_step": round(enqueue_us / args.steps, 1),
                    "queued": bool(hold_us >= enqueue_us)})
    return dt, us, dom


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        n = 1
    return int(n)


# ---------------------------------------------------------------- workloads
def run_decode7b(args, torch, B, W):
    """The default line.

    value / roofline: the FP8 W8A8 block GEMM of the 7B-class decode FFN
    up/gate layer (A [64, 3584], Wt [37888, 3584]), the decode-shape half of
    the metric, as algorithmic GB/s of the GEMM itself.  One step is one
    decode pass of the layer: FP8 token-group quantization of the activation
    batch, then the GEMM against the layer's FP8 weight.  The weight was
    quantized before (a rollout quantizes it once per training step and
    decodes with it many times), and five copies of it alternate so that no
    step finds it in the 256 MB last-level cache.  HIP events on the launch
    stream around the GEMM calls of the timed steps give its duration.

    prefill: the other half of the metric, the FP8 GEMM of the 32B-class
    prefill up/gate layer (M 8192, N 27648, K 5120) in TFLOP/s against the
    FP8 peak, with its own CPU baseline; the down projection beside it.

    requant_step: the whole per-step path at this shape (FP8 block
    re-quantization of the bf16 weight, activation quantization, GEMM, and
    the INT8 per-channel variant of all three), as before.
    """
    M, N, K = 64, 37888, 3584
    dev = torch.device("cuda:0")
    inputs = []
    for seed in (0, 1):
        p = W.gemm_problem(M, N, K, True, seed=seed)
        inputs.append(dict(A=torch.from_numpy(p["A"].view(np.int16)).cuda(),
                           Wt=torch.from_numpy(p["Wt"].view(np.int16)).cuda()))
    w8 = B.fp8_weight_block_quant(inputs[0]["Wt"])
    copies = _cold_copies(torch, lambda i: (w8[0].clone(), w8[1].clone()), N * K)
    # One activation batch per timed step (the decode of K tokens' worth of
    # batches), quantized in the step.
    nsteps = max(1, args.steps)
    aq8 = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in range(nsteps)]
    sa8 = [torch.empty((M, K // 128), dtype=torch.float32, device=dev) for _ in range(nsteps)]
    c8 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    gbytes = gemm_bytes(M, N, K, M * (K // 128), cdiv(N, 128) * (K // 128))
    abytes = quant_bytes(M, K, M * (K // 128))

    def quant(i):
        B.fp8_act_token_quant(inputs[i % 2]["A"], out=aq8[i % nsteps], scale=sa8[i % nsteps])

    def gemm(i):
        wq, sw = copies[i % len(copies)]
        B.w8a8_block_gemm(aq8[i % nsteps], sa8[i % nsteps], wq, sw, out=c8)

    t0 = time.perf_counter()
    for i in range(args.warmup):
        quant(i)
        gemm(i)
    host_us = (time.perf_counter() - t0) * 1e6 / max(1, args.warmup)
    torch.cuda.synchronize()
    # Timed region: the K steps' activation quantizations, then their K GEMMs
    # back to back (each on the next of the cold weight copies); a pair of HIP
    # events on the launch stream brackets each of the two runs, so the GEMM's
    # average launch duration includes the dispatch gap between launches.
    # The runs start behind a hold of the stream (hold_stream): the ~4 us
    # quantizations are shorter than the host's calls, and would otherwise
    # be timed at the host's pace.  The step time is the GPU time of the two
    # runs.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    hold_stream(torch, 4 * host_us * args.steps + 500, mark=None)
    ev[0].record()
    for i in range(args.steps):
        quant(i)
    ev[1].record()
    for i in range(args.steps):
        gemm(i)
    ev[2].record()
    torch.cuda.synchronize()
    dt = ev[0].elapsed_time(ev[2]) * 1e-3 / args.steps
    q_us = ev[0].elapsed_time(ev[1]) * 1e3 / args.steps
    g_us = ev[1].elapsed_time(ev[2]) * 1e3 / args.steps
    achieved = gbytes / g_us / 1e3
    roofline = {"bound": "hbm", "kernel": "w8a8_block_gemm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "us_per_launch": round(g_us, 2),
                "traffic": measured_traffic("w8a8_block_gemm", "decode7b_upgate")}
    act = {"fp8_act_token_quant": {"us_per_launch": round(q_us, 2),
                                   "GB/s": round(abytes / q_us / 1e3, 1)}}
    req = requant_step_decode7b(args, torch, B, W, inputs)
    line = {
        "metric": METRIC, "value": round(achieved, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8e4m3", "data": "synthetic",
        "config": {"workload": "decode7b_upgate", "M": M, "N": N, "K": K,
                   "value_is": "fp8 W8A8 block GEMM algorithmic GB/s: HIP events around the "
                               "timed steps' GEMMs launched back to back, cold weights",
                   "step": "fp8 A group quant + fp8 W8A8 block GEMM (weight quantized before)",
                   "gemm_algorithmic_bytes": gbytes,
                   "step_algorithmic_bytes": gbytes + abytes},
        "roofline": roofline, "step_kernels": act,
    }
    line["prefill"] = prefill_upgate_line(args, torch, B, W)
    line["requant_step"] = req
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode_gemm(W, gbytes)
        line["prefill"]["cpu_baseline"] = cpu_baseline_prefill(W)
    return line


def requant_step_decode7b(args, torch, B, W, inputs):
    """The six calls of one full per-step pass at the 7B decode shape (FP8
    and INT8 weight re-quantization, activation quantization and GEMM), the
    two input sets alternating; per-kernel durations from an instrumented
    pass (event pair around every call)."""
    M, N, K = 64, 37888, 3584
    dev = torch.device("cuda:0")
    outs = []
    for _ in inputs:
        outs.append(dict(
            wq8=torch.empty((N, K), dtype=torch.uint8, device=dev),
            sw8=torch.empty((cdiv(N, 128), K // 128), dtype=torch.float32, device=dev),
            aq8=torch.empty((M, K), dtype=torch.uint8, device=dev),
            sa8=torch.empty((M, K // 128), dtype=torch.float32, device=dev),
            c8=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
            wqi=torch.empty((N, K), dtype=torch.int8, device=dev),
            swi=torch.empty((N,), dtype=torch.float32, device=dev),
            aqi=torch.empty((M, K), dtype=torch.int8, device=dev),
            sai=torch.empty((M,), dtype=torch.float32, device=dev),
            ci=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    work = {
        "fp8_weight_block_quant": quant_bytes(N, K, cdiv(N, 128) * (K // 128)),
        "fp8_act_token_quant": quant_bytes(M, K, M * (K // 128)),
        "w8a8_block_gemm": gemm_bytes(M, N, K, M * (K // 128), cdiv(N, 128) * (K // 128)),
        "int8_weight_channel_quant": quant_bytes(N, K, N),
        "int8_act_token_quant": quant_bytes(M, K, M),
        "w8a8_int8_channel_gemm": gemm_bytes(M, N, K, M, N),
    }
    step_bytes = sum(work.values())

    def step(i, timer=None):
        s, o = inputs[i % 2], outs[i % 2]
        t = timer.run if timer else (lambda _n, f: f())
        t("fp8_weight_block_quant", lambda: B.fp8_weight_block_quant(s["Wt"], out=o["wq8"], scale=o["sw8"]))
        t("fp8_act_token_quant", lambda: B.fp8_act_token_quant(s["A"], out=o["aq8"], scale=o["sa8"]))
        t("w8a8_block_gemm", lambda: B.w8a8_block_gemm(o["aq8"], o["sa8"], o["wq8"], o["sw8"], out=o["c8"]))
        t("int8_weight_channel_quant", lambda: B.int8_weight_channel_quant(s["Wt"], out=o["wqi"], scale=o["swi"]))
        t("int8_act_token_quant", lambda: B.int8_act_token_quant(s["A"], out=o["aqi"], scale=o["sai"]))
        t("w8a8_int8_channel_gemm", lambda: B.w8a8_int8_channel_gemm(o["aqi"], o["sai"], o["wqi"], o["swi"], out=o["ci"]))

    sub = argparse.Namespace(steps=min(args.steps, 20), warmup=max(1, min(args.warmup, 3)))
    dt, us, dom = timed_steps(torch, step, sub)
    kernels = {k: {"us": round(us[k], 2), "algorithmic_bytes": work[k],
                   "GB/s": round(work[k] / us[k] / 1e3, 1)} for k in work}
    return {"steps": sub.steps, "ms_per_step": round(dt * 1e3, 4),
            "GB/s": round(step_bytes / dt / 1e9, 1), "step_algorithmic_bytes": step_bytes,
            "step": "fp8 W block quant + fp8 A group quant + fp8 W8A8 GEMM + int8 W channel "
                    "quant + int8 A token quant + int8 W8A8 GEMM (the GEMMs read the codes the "
                    "same step wrote)",
            "dominant": dom, "kernels": kernels}


def prefill_upgate_line(args, torch, B, W):
    """FP8 W8A8 block GEMM of the 32B-class prefill up/gate layer (M 8192,
    N 27648, K 5120) in TFLOP/s: one pair of HIP events around steps / 4
    (at least 10) launches back to back, against the 5.0 PFLOP/s dense FP8
    peak; the down projection (N 5120, K 27648) beside it."""
    out = {}
    for which, (N, K) in (("upgate", (27648, 5120)), ("down", (5120, 27648))):
        p = W.gemm_problem(8192, N, K, True, seed=0, down=which == "down")
        a = torch.from_numpy(p["A"].view(np.int16)).cuda()
        w = torch.from_numpy(p["Wt"].view(np.int16)).cuda()
        aq, sa = B.fp8_act_token_quant(a)
        wq, sw = B.fp8_weight_block_quant(w)
        del a, w
        c = torch.empty((8192, N), dtype=torch.bfloat16, device="cuda:0")
        for _ in range(max(2, args.warmup)):
            B.w8a8_block_gemm(aq, sa, wq, sw, out=c)
        n = max(10, args.steps // 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            B.w8a8_block_gemm(aq, sa, wq, sw, out=c)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        tf = 2 * 8192 * N * K / us / 1e6
        out[which] = {"M": 8192, "N": N, "K": K, "us": round(us, 2), "TFLOP/s": round(tf, 1),
                      "frac": round(tf / FP8_PEAK_TFLOPS, 4), "launches": n}
        del aq, sa, wq, sw, c
    up = out["upgate"]
    return {"workload": "prefill32b up/gate: A [8192, 5120] x Wt [27648, 5120], FP8 blocks",
            "value": up["TFLOP/s"], "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "kernel": "w8a8_block_gemm",
                         "achieved": up["TFLOP/s"], "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": up["frac"],
                         "traffic": measured_traffic("w8a8_block_gemm", "prefill32b")},
            "gemms": out}


def cpu_cores():
    return {"blas_threads": cpu_threads(), "os_cpu_count": os.cpu_count()}


def _repeat_timed(fn, min_seconds=8.0, max_reps=50):
    """Run fn until min_seconds of it have been timed (at least twice):
    (repeats, total seconds).  One call of the oracle GEMM takes 0.5-2 s,
    short enough for the host's timer noise to show."""
    reps, total = 0, 0.0
    while reps < 2 or (total < min_seconds and reps < max_reps):
        t0 = time.perf_counter()
        fn()
        total += time.perf_counter() - t0
        reps += 1
    return reps, total


def cpu_baseline_decode_gemm(W, gbytes):
    """The oracle, as it stands, on the same GEMM: the FP8 GEMM of the full
    A [64, 3584] against the full FP8 weight [37888, 3584] (fp64 BLAS over the
    decoded codes), in the line's unit; the operands are quantized by the
    oracle first, outside the timed part."""
    from oracle import gemm, quant
    M, N, K = 64, 37888, 3584
    p = W.gemm_problem(M, N, K, True, seed=0)
    wq, sw = quant.fp8_weight_block_quant(p["Wt"])
    aq, sa = quant.fp8_act_token_quant(p["A"])
    reps, total = _repeat_timed(lambda: gemm.round_bf16(gemm.w8a8_block_gemm(aq, sa, wq, sw)))
    cores = cpu_cores()
    return {"value": round(reps * gbytes / total / 1e9, 4), "unit": "GB/s",
            "cores": cores["blas_threads"], "os_cpu_count": cores["os_cpu_count"],
            "kind": "oracle", "seconds": round(total, 2), "repeats": reps,
            "sample": f"the whole GEMM, {reps} times: A [64, 3584] x Wt [37888, 3584] FP8 "
                      "codes and scales, rounded to bf16; fp64 BLAS with the host's BLAS threads"}


def cpu_baseline_prefill(W, rows=512):
    """The oracle on a row sample of the prefill up/gate GEMM: `rows` token
    rows of A [8192, 5120] against the full FP8 weight [27648, 5120], in
    TFLOP/s of that sample (operands quantized by the oracle first, outside
    the timed part)."""
    from oracle import gemm, quant
    N, K = 27648, 5120
    p = W.gemm_problem(8192, N, K, True, seed=0)
    wq, sw = quant.fp8_weight_block_quant(p["Wt"])
    aq, sa = quant.fp8_act_token_quant(p["A"][:rows])
    reps, total = _repeat_timed(lambda: gemm.round_bf16(gemm.w8a8_block_gemm(aq, sa, wq, sw)))
    cores = cpu_cores()
    return {"value": round(reps * 2 * rows * N * K / total / 1e12, 5), "unit": "TFLOP/s",
            "cores": cores["blas_threads"], "os_cpu_count": cores["os_cpu_count"],
            "kind": "oracle", "seconds": round(total, 2), "repeats": reps,
            "sample": f"the first {rows} of 8192 token rows against the full weight "
                      f"[27648, 5120], {reps} times; fp64 BLAS with the host's BLAS threads"}


def _cold_copies(torch, make, nbytes, budget=600 << 20):
    """Enough copies of a tensor set that cycling through them cannot be
    served by the 256 MB last-level cache."""
    n = max(2, -(-budget // max(1, nbytes)))
    return [make(i) for i in range(min(n, 64))]


def run_decode32b(args, torch, B, W):
    A, Wt = W.decode_sweep(seed=0)
    wdev = torch.from_numpy(Wt.view(np.int16)).cuda()
    w8 = B.fp8_weight_block_quant(wdev)
    wi = B.int8_weight_channel_quant(wdev)
    N, K = Wt.shape
    copies8 = _cold_copies(torch, lambda i: (w8[0].clone(), w8[1].clone()), N * K)
    copiesi = _cold_copies(torch, lambda i: (wi[0].clone(), wi[1].clone()), N * K)
    del wdev
    res = {}
    for M in W.DECODE_SWEEP_M:
        a = torch.from_numpy(A[:M].copy().view(np.int16)).cuda()
        aq8, sa8 = B.fp8_act_token_quant(a)
        aqi, sai = B.int8_act_token_quant(a)
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        for name, cp, fn, aq, sa, nws, nas in (
                ("w8a8_block_gemm", copies8, B.w8a8_block_gemm, aq8, sa8, (N // 128) * (K // 128), M * (K // 128)),
                ("w8a8_int8_channel_gemm", copiesi, B.w8a8_int8_channel_gemm, aqi, sai, N, M)):
            for i in range(args.warmup):
                fn(aq, sa, cp[i % len(cp)][0], cp[i % len(cp)][1], out=c)
            timer = Timer(torch)
            for i in range(args.steps):
                wq, sw = cp[i % len(cp)]
                timer.run(name, lambda: fn(aq, sa, wq, sw, out=c))
            torch.cuda.synchronize()
            us = timer.avg_us()[name]
            by = gemm_bytes(M, N, K, nas, nws)
            res[f"{name}/M{M}"] = {"us": round(us, 2), "GB/s": round(by / us / 1e3, 1),
                                   "TFLOP/s": round(2 * M * N * K / us / 1e6, 2),
                                   "hbm_frac": round(by / us / 1e3 / HBM_PEAK_GBS, 4)}
    worst = min(v["GB/s"] for k, v in res.items() if k.startswith("w8a8_block_gemm"))
    return {"metric": METRIC, "value": worst, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "higher_is_better": True, "vs_baseline": None,
            "dtype": "fp8e4m3+int8", "data": "synthetic",
            "config": {"workload": "decode32b_sweep", "N": N, "K": K,
                       "value_is": "lowest fp8 GEMM GB/s over M"},
            "kernels": res}


def run_prefill32b(args, torch, B, W):
    res = {}
    for which, (N, K) in (("upgate", (27648, 5120)), ("down", (5120, 27648))):
        p = W.gemm_problem(8192, N, K, True, seed=0, down=which == "down")
        a = torch.from_numpy(p["A"].view(np.int16)).cuda()
        w = torch.from_numpy(p["Wt"].view(np.int16)).cuda()
        aq8, sa8 = B.fp8_act_token_quant(a)
        wq8, sw8 = B.fp8_weight_block_quant(w)
        aqi, sai = B.int8_act_token_quant(a)
        wqi, swi = B.int8_weight_channel_quant(w)
        c = torch.empty((8192, N), dtype=torch.bfloat16, device="cuda:0")
        flops = 2 * 8192 * N * K
        for name, fn, args_ in (("w8a8_block_gemm", B.w8a8_block_gemm, (aq8, sa8, wq8, sw8)),
                                ("w8a8_int8_channel_gemm", B.w8a8_int8_channel_gemm, (aqi, sai, wqi, swi)),
                                ("fp8_act_token_quant", None, None)):
            timer = Timer(torch)
            if fn is None:
                for i in range(args.warmup):
                    B.fp8_act_token_quant(a, out=aq8, scale=sa8)
                for i in range(args.steps):
                    timer.run(name, lambda: B.fp8_act_token_quant(a, out=aq8, scale=sa8))
                torch.cuda.synchronize()
                us = timer.avg_us()[name]
                by = quant_bytes(8192, K, 8192 * (K // 128))
                res[f"{name}/{which}"] = {"us": round(us, 2), "GB/s": round(by / us / 1e3, 1)}
                continue
            for i in range(args.warmup):
                fn(*args_, out=c)
            for i in range(args.steps):
                timer.run(name, lambda: fn(*args_, out=c))
            torch.cuda.synchronize()
            us = timer.avg_us()[name]
            tf = flops / us / 1e6
            res[f"{name}/{which}"] = {"us": round(us, 2), "TFLOP/s": round(tf, 1),
                                      "peak_frac": round(tf / FP8_PEAK_TFLOPS, 4)}
        del a, w, c
    up = res["w8a8_block_gemm/upgate"]
    line = {"metric": METRIC, "value": up["TFLOP/s"], "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "vs_baseline": None, "dtype": "fp8e4m3+int8", "data": "synthetic",
            "config": {"workload": "prefill32b", "M": 8192,
                       "value_is": "fp8 up/gate GEMM M8192 N27648 K5120"},
            "roofline": {"bound": "mfma", "kernel": "w8a8_block_gemm", "achieved": up["TFLOP/s"],
                         "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": up["peak_frac"],
                         "traffic": measured_traffic("w8a8_block_gemm", "prefill32b")},
            "kernels": res}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(W)
    return line


def run_stack32b(args, torch, B, W):
    """Per-step re-quantization of a 32B-class layer's seven weights (q, k, v,
    o, gate, up, down; 487.6 M elements, 975 MB of bf16): all seven in one
    FP8 launch (fp8_weight_block_quant_multi) and in one INT8 launch
    (int8_weight_channel_quant_multi) per step; the 1.46 GB each launch
    moves is far beyond the 256 MB last-level cache.  The one-weight calls
    are timed beside them (`per_weight`: seven launches per format)."""
    ws = [torch.from_numpy(W.stack_layer(name, 0).view(np.int16)).cuda()
          for name, _, _ in W.STACK_32B]
    o8 = B.fp8_weight_block_quant_multi(ws)
    oi = B.int8_weight_channel_quant_multi(ws)

    def step(_i, timer=None):
        t = timer.run if timer else (lambda _n, f: f())
        t("fp8_weight_block_quant_multi", lambda: B.fp8_weight_block_quant_multi(ws, outs=o8))
        t("int8_weight_channel_quant_multi", lambda: B.int8_weight_channel_quant_multi(ws, outs=oi))

    dt, us, _ = timed_steps(torch, step, args)
    elems = sum(N * K for _, N, K in W.STACK_32B)
    b8 = sum(quant_bytes(N, K, cdiv(N, 128) * cdiv(K, 128)) for _, N, K in W.STACK_32B)
    bi = sum(quant_bytes(N, K, N) for _, N, K in W.STACK_32B)

    def single(_i, timer=None):
        for w, (q8, s8), (qi, si) in zip(ws, o8, oi):
            f8 = lambda: B.fp8_weight_block_quant(w, out=q8, scale=s8)
            fi = lambda: B.int8_weight_channel_quant(w, out=qi, scale=si)
            if timer:
                timer.run("fp8_weight_block_quant", f8)
                timer.run("int8_weight_channel_quant", fi)
            else:
                f8(); fi()
    sub = argparse.Namespace(steps=min(args.steps, 10), warmup=1)
    dts, uss, _ = timed_steps(torch, single, sub)
    per8 = uss["fp8_weight_block_quant"] * len(ws)
    peri = uss["int8_weight_channel_quant"] * len(ws)
    u8, ui = us["fp8_weight_block_quant_multi"], us["int8_weight_channel_quant_multi"]
    dom, dom_us, dom_b = ("fp8_weight_block_quant_multi", u8, b8) if u8 >= ui else \
        ("int8_weight_channel_quant_multi", ui, bi)
    return {"metric": METRIC, "value": round((b8 + bi) / dt / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 3),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "fp8e4m3+int8", "data": "synthetic",
            "config": {"workload": "stack32b_requant", "elements": elems,
                       "step": "fp8 multi-weight block quant + int8 multi-weight channel quant "
                               "of the seven weights"},
            "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dom_b / dom_us / 1e3, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dom_b / dom_us / 1e3 / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(dom, "stack32b_requant")},
            "kernels": {"fp8_weight_block_quant_multi": {"us": round(u8, 1), "GB/s": round(b8 / u8 / 1e3, 1)},
                        "int8_weight_channel_quant_multi": {"us": round(ui, 1), "GB/s": round(bi / ui / 1e3, 1)}},
            "per_weight": {"ms_per_step": round(dts * 1e3, 3),
                           "fp8_weight_block_quant x7": {"us": round(per8, 1), "GB/s": round(b8 / per8 / 1e3, 1)},
                           "int8_weight_channel_quant x7": {"us": round(peri, 1), "GB/s": round(bi / peri / 1e3, 1)}}}


def run_stack_gemm(args, torch, B, W):
    """The W8A8 GEMMs of one 32B-shaped layer stack at decode batch sizes:
    for M in (1, 64), the FP8 block-scaled and the INT8 per-channel GEMM of
    each of the seven weights (q, k, v, o, gate, up, down; 487 MB of 8-bit
    weights per pass, so no GEMM finds its weight in the 256 MB last-level
    cache).  value: algorithmic bytes of the whole pass / its time."""
    layers = []
    for name, N, K in W.STACK_32B:
        w = torch.from_numpy(W.stack_layer(name, 0).view(np.int16)).cuda()
        layers.append((name, N, K, B.fp8_weight_block_quant(w), B.int8_weight_channel_quant(w)))
        del w
    res, total_bytes, total_s = {}, 0, 0.0
    for M in (1, 64):
        acts = {}
        for name, N, K, _, _ in layers:
            if K not in acts:
                a = torch.from_numpy(W.activation(M, K, 0).view(np.int16)).cuda()
                acts[K] = (B.fp8_act_token_quant(a), B.int8_act_token_quant(a))
        outs = {name: torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
                for name, N, K, _, _ in layers}
        work = {}
        for name, N, K, _, _ in layers:
            work[f"w8a8_block_gemm/{name}/M{M}"] = gemm_bytes(M, N, K, M * (K // 128),
                                                             cdiv(N, 128) * (K // 128))
            work[f"w8a8_int8_channel_gemm/{name}/M{M}"] = gemm_bytes(M, N, K, M, N)

        def step(_i, timer=None, M=M, acts=acts, outs=outs):
            t = timer.run if timer else (lambda _n, f: f())
            for name, N, K, (wq, sw), (wqi, swi) in layers:
                (aq, sa), (aqi, sai) = acts[K]
                c = outs[name]
                t(f"w8a8_block_gemm/{name}/M{M}", lambda: B.w8a8_block_gemm(aq, sa, wq, sw, out=c))
                t(f"w8a8_int8_channel_gemm/{name}/M{M}",
                  lambda: B.w8a8_int8_channel_gemm(aqi, sai, wqi, swi, out=c))

        dt, us, _ = timed_steps(torch, step, args)
        for k, v in us.items():
            res[k] = {"us": round(v, 2), "GB/s": round(work[k] / v / 1e3, 1),
                      "hbm_frac": round(work[k] / v / 1e3 / HBM_PEAK_GBS, 4)}
        total_bytes += sum(work.values())
        total_s += dt
    dom = max(res, key=lambda k: res[k]["us"])   # the longest call of the pass
    return {"metric": METRIC, "value": round(total_bytes / total_s / 1e9, 1), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(total_s * 1e3, 3), "higher_is_better": True, "vs_baseline": None,
            "dtype": "fp8e4m3+int8", "data": "synthetic",
            "config": {"workload": "stack32b_gemm", "M": [1, 64],
                       "layers": [list(x) for x in W.STACK_32B],
                       "value_is": "algorithmic bytes of all 28 GEMM calls / their time"},
            "roofline": {"bound": "hbm", "kernel": dom, "achieved": res[dom]["GB/s"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": res[dom]["hbm_frac"],
                         "traffic": None},
            "kernels": res}


def run_kv32b(args, torch, B, W):
    """FP8 KV cache of a 32B-class layer for a 16,384-token prefill: per
    step, the K and V rows written into a 65,536-slot cache (16-slot pages
    in random order) with the scales the previous step calibrated, and the
    next step's scales recalibrated from them.

    value / roofline: the step as one call for K and V
    (fp8_kv_cache_write_recalibrate_multi), algorithmic bytes (both
    tensors' rows read once, their codes written, the slot mapping, the
    scales) per second.  `forms` times the same step as one one-pass call
    per tensor, and as the separate recalibration and write calls (which
    read the rows twice), against the same algorithmic bytes."""
    cfg = W.KV_32B
    T, C, S = cfg["T"], cfg["C"], cfg["num_slots"]
    kb, vb = W.kv_rows(T, C, 0, "K"), W.kv_rows(T, C, 0, "V")
    k = torch.from_numpy(kb.view(np.int16)).cuda()
    v = torch.from_numpy(vb.view(np.int16)).cuda()
    slots_np = W.kv_slot_mapping(T, S, cfg["page"], 0)
    slots = torch.from_numpy(slots_np).cuda()
    kc = torch.zeros((S, C), dtype=torch.uint8, device="cuda:0")
    vc = torch.zeros_like(kc)
    ks = torch.empty(1, dtype=torch.float32, device="cuda:0")
    vs = torch.empty_like(ks)
    B.fp8_kv_scale_recalibrate(k, out=ks)
    B.fp8_kv_scale_recalibrate(v, out=vs)
    kws = torch.empty(2 * B.KV_RECAL_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    step_bytes = 2 * (3 * T * C + 8) + 8 * T          # rows read, codes written, scales; slots once

    def multi_step(_i, timer=None):
        fn = lambda: B.fp8_kv_cache_write_recalibrate_multi([k, v], slots, [ks, vs], [kc, vc],
                                                            new_scales=[ks, vs], workspace=kws)
        timer.run("fp8_kv_cache_write_recalibrate_multi", fn) if timer else fn()

    def per_tensor_step(_i, timer=None):
        calls = [("fp8_kv_cache_write_recalibrate",
                  lambda: B.fp8_kv_cache_write_recalibrate(k, slots, ks, kc, new_scale=ks,
                                                           workspace=kws)),
                 ("fp8_kv_cache_write_recalibrate",
                  lambda: B.fp8_kv_cache_write_recalibrate(v, slots, vs, vc, new_scale=vs,
                                                           workspace=kws))]
        for name, fn in calls:
            timer.run(name, fn) if timer else fn()

    def separate_step(_i, timer=None):
        calls = [("fp8_kv_scale_recalibrate", lambda: B.fp8_kv_scale_recalibrate(k, out=ks)),
                 ("fp8_kv_scale_recalibrate", lambda: B.fp8_kv_scale_recalibrate(v, out=vs)),
                 ("fp8_kv_cache_write", lambda: B.fp8_kv_cache_write(k, slots, ks, kc)),
                 ("fp8_kv_cache_write", lambda: B.fp8_kv_cache_write(v, slots, vs, vc))]
        for name, fn in calls:
            timer.run(name, fn) if timer else fn()

    dt, us, _ = timed_steps(torch, multi_step, args)
    pdt, pus, _ = timed_steps(torch, per_tensor_step, args)
    sdt, sus, _ = timed_steps(torch, separate_step, args)
    m_us = us["fp8_kv_cache_write_recalibrate_multi"]
    b_recal = 2 * T * C + 4
    b_write = 3 * T * C + 8 * T + 4
    b_one = 3 * T * C + 8 * T + 8
    line = {"metric": METRIC, "value": round(step_bytes / dt / 1e9, 1), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(dt * 1e3, 4), "higher_is_better": True, "vs_baseline": None,
            "dtype": "fp8e4m3", "data": "synthetic",
            "config": {"workload": "kv32b_prefill", "tokens": T, "row": C, "slots": S,
                       "step": "fp8_kv_cache_write_recalibrate_multi for K and V (write with "
                               "the previous step's scales, recalibrate the next from the same "
                               "rows)", "step_algorithmic_bytes": step_bytes},
            "roofline": {"bound": "hbm", "kernel": "fp8_kv_cache_write_recalibrate_multi",
                         "achieved": round(step_bytes / m_us / 1e3, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(step_bytes / m_us / 1e3 / HBM_PEAK_GBS, 4),
                         "us_per_launch": round(m_us, 2),
                         "traffic": measured_traffic("fp8_kv_cache_write_recalibrate_multi",
                                                     "kv32b_prefill")},
            "forms": {
                "per_tensor_calls": {
                    "ms_per_step": round(pdt * 1e3, 4),
                    "GB/s": round(step_bytes / pdt / 1e9, 1),
                    "fp8_kv_cache_write_recalibrate": {
                        "us": round(pus["fp8_kv_cache_write_recalibrate"], 2),
                        "algorithmic_bytes": b_one,
                        "traffic": measured_traffic("fp8_kv_cache_write_recalibrate",
                                                    "kv32b_prefill")}},
                "separate_calls": {
                    "ms_per_step": round(sdt * 1e3, 4),
                    "GB/s": round(step_bytes / sdt / 1e9, 1),
                    "fp8_kv_scale_recalibrate": {
                        "us": round(sus["fp8_kv_scale_recalibrate"], 2), "algorithmic_bytes": b_recal,
                        "GB/s": round(b_recal / sus["fp8_kv_scale_recalibrate"] / 1e3, 1)},
                    "fp8_kv_cache_write": {
                        "us": round(sus["fp8_kv_cache_write"], 2), "algorithmic_bytes": b_write,
                        "GB/s": round(b_write / sus["fp8_kv_cache_write"] / 1e3, 1),
                        "traffic": measured_traffic("fp8_kv_cache_write", "kv32b_prefill")}},
                "speedup_vs_separate_calls": round(sdt / dt, 3)}}
    if not args.no_cpu_baseline:
        from oracle import kv as okv
        cache0 = np.zeros((S, C), np.uint8)
        s_old = {id(kb): okv.kv_scale(kb), id(vb): okv.kv_scale(vb)}
        t0 = time.perf_counter()
        for xb in (kb, vb):
            okv.kv_cache_write(cache0, xb, slots_np, s_old[id(xb)])
            okv.kv_scale(xb)
        ct = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(step_bytes / ct / 1e9, 3), "unit": "GB/s",
                                "cores": cpu_threads(), "os_cpu_count": os.cpu_count(), "kind": "oracle",
                                "sample": "one whole step (K and V: cache write with the earlier "
                                          "scale and the new scale)"}
    return line


def grouped_bytes(counts, N, K):
    """Rows and their scales, the weights and scales of every expert that
    has rows, the bf16 output and the row offsets."""
    counts = np.asarray(counts)
    M, E, KB = int(counts.sum()), len(counts), K // 128
    active = int(np.count_nonzero(counts))
    return (M * K + 4 * M * KB + active * (N * K + 4 * cdiv(N, 128) * KB) + 2 * M * N
            + 8 * (E + 1))


def run_moe_decode(args, torch, B, W):
    """One decode step of a mixture-of-experts layer (128 experts, top-8
    routing of 128 tokens, expert N = 1536, K = 2048): FP8 block quant of
    every expert's weight, FP8 group quant of the routed rows, and the
    grouped W8A8 GEMM over all experts in one launch."""
    cfg = W.MOE_DECODE
    E, N, K = cfg["E"], cfg["N"], cfg["K"]
    counts = W.moe_routing(cfg["tokens"], E, cfg["topk"], seed=0)
    p = W.moe_problem(counts, N, K, seed=0)
    M, KB, NB = p["M"], K // 128, cdiv(N, 128)
    dev = torch.device("cuda:0")
    A = torch.from_numpy(p["A"].view(np.int16)).to(dev)
    Wt = torch.from_numpy(p["Wt"].reshape(E * N, K).view(np.int16)).to(dev)
    offsets = torch.from_numpy(p["offsets"]).to(dev)
    hint = int(counts.max())
    wq = torch.empty((E * N, K), dtype=torch.uint8, device=dev)
    sw = torch.empty((E * NB, KB), dtype=torch.float32, device=dev)
    aq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, KB), dtype=torch.float32, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    work = {
        "fp8_weight_block_quant": quant_bytes(E * N, K, E * NB * KB),
        "fp8_act_token_quant": quant_bytes(M, K, M * KB),
        "w8a8_block_gemm_grouped": grouped_bytes(counts, N, K),
    }
    step_bytes = sum(work.values())

    def step(_i, timer=None):
        t = timer.run if timer else (lambda _n, f: f())
        t("fp8_weight_block_quant", lambda: B.fp8_weight_block_quant(Wt, out=wq, scale=sw))
        t("fp8_act_token_quant", lambda: B.fp8_act_token_quant(A, out=aq, scale=sa))
        t("w8a8_block_gemm_grouped", lambda: B.w8a8_block_gemm_grouped(
            aq, sa, wq.view(E, N, K), sw.view(E, NB, KB), offsets, hint, out=c))

    dt, us, dom = timed_steps(torch, step, args)
    kernels = {k: {"us": round(us[k], 2), "algorithmic_bytes": work[k],
                   "GB/s": round(work[k] / us[k] / 1e3, 1)} for k in work}
    achieved = work[dom] / us[dom] / 1e3
    line = {
        "metric": METRIC, "value": round(step_bytes / dt / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8e4m3", "data": "synthetic",
        "config": {"workload": "moe_decode", "experts": E, "topk": cfg["topk"],
                   "tokens": cfg["tokens"], "rows": M, "N": N, "K": K,
                   "rows_per_expert": [int(counts.min()), int(counts.max())],
                   "step": "fp8 W block quant (all experts) + fp8 A group quant + grouped "
                           "fp8 W8A8 GEMM",
                   "step_algorithmic_bytes": step_bytes},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(dom, "moe_decode")},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        from oracle import gemm, quant
        ns = E                                  # the whole step (about 10 s on 16 cores)
        sub = counts[:ns]
        r1 = int(sub.sum())
        t0 = time.perf_counter()
        wqs = [quant.fp8_weight_block_quant(p["Wt"][e]) for e in range(ns)]
        aqs, sas = quant.fp8_act_token_quant(p["A"][:r1])
        gemm.w8a8_block_gemm_grouped(aqs, sas, np.stack([w for w, _ in wqs]),
                                     np.stack([x for _, x in wqs]), p["offsets"][:ns + 1])
        ct = time.perf_counter() - t0
        sample = (quant_bytes(ns * N, K, ns * NB * KB) + quant_bytes(r1, K, r1 * KB)
                  + grouped_bytes(sub, N, K))
        line["cpu_baseline"] = {"value": round(sample / ct / 1e9, 4), "unit": "GB/s",
                                "cores": cpu_threads(), "os_cpu_count": os.cpu_count(), "kind": "oracle", "seconds": round(ct, 2),
                                "sample": f"one whole step: weight quant of all {ns} experts, "
                                          f"quant of the {r1} routed rows, the grouped GEMM"}
    return line


def run_att(args, torch, B, W):
    """Decode attention over the FP8 KV cache of a 32B-class layer (40 query
    heads over 8 KV heads of 128): 64 sequences of 1024-8192 cached tokens
    in 16-slot pages taken in random order (604 MB of K and V codes, so no
    step finds them in the 256 MB last-level cache)."""
    cfg = W.ATT_32B
    Bn, Hq, Hkv, D, page = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["page"]
    lens = W.att_lengths(Bn, cfg["min_len"], cfg["max_len"], 0)
    table, num_slots = W.att_block_table(lens, page, 0)
    q_np = W.att_query(Bn, Hq, D, 0)
    kc_np = W.att_random_codes(num_slots, Hkv * D, 0)
    vc_np = W.att_random_codes(num_slots, Hkv * D, 1)
    dev = torch.device("cuda:0")
    q = torch.from_numpy(q_np.reshape(Bn, -1).view(np.int16)).to(dev).view(Bn, Hq, D)
    kc, vc = torch.from_numpy(kc_np).to(dev), torch.from_numpy(vc_np).to(dev)
    tb, sl = torch.from_numpy(table).to(dev), torch.from_numpy(lens).to(dev)
    sq = B.fp8_kv_scale_recalibrate(q.view(Bn, -1))
    sk = torch.tensor([2.0 ** -12], dtype=torch.float32, device=dev)
    sv = torch.tensor([2.0 ** -8], dtype=torch.float32, device=dev)
    out = torch.empty((Bn, Hq, D), dtype=torch.bfloat16, device=dev)
    tokens = int(lens.sum())

    def att_work(ls):
        return (2 * int(ls.sum()) * Hkv * D + 4 * len(ls) * Hq * D
                + 4 * int(((ls + page - 1) // page).sum()) + 4 * len(ls))

    work = att_work(lens)
    # the batch split over the CUs, with the workspace the library asks for
    wsb = B.attention_workspace_bytes(Bn, Hq, Hkv, D)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=dev) if wsb else None

    def step(_i, timer=None):
        f = lambda: B.fp8_kv_decode_attention(q, sq, kc, vc, sk, sv, tb, sl, Hkv, page, out=out,
                                              workspace=ws)
        timer.run("fp8_kv_decode_attention", f) if timer else f()

    dt, us, dom = timed_steps(torch, step, args)

    # Long-tail batches (the first b sequences of the same cache): both launch
    # forms, median of 20 event-timed calls each.
    def median_us(f, n=20):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for a, e in ev:
            a.record()
            f()
            e.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(e) * 1e3 for a, e in ev]))

    tail = {}
    for b in (1, 2, 8, Bn):
        wb = B.attention_workspace_bytes(b, Hq, Hkv, D)
        wt = torch.empty((wb,), dtype=torch.uint8, device=dev) if wb else None
        ob = out[:b]
        row = {}
        for name, w in (("split", wt), ("one_pass", None)):
            t = median_us(lambda: B.fp8_kv_decode_attention(q[:b], sq, kc, vc, sk, sv, tb[:b],
                                                            sl[:b], Hkv, page, out=ob,
                                                            workspace=w))
            row[name] = {"us": round(t, 1), "GB/s": round(att_work(lens[:b]) / t / 1e3, 1)}
        tail[f"B{b}"] = row
    line = {"metric": METRIC, "value": round(work / dt / 1e9, 1), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(dt * 1e3, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8e4m3", "data": "synthetic",
            "config": {"workload": "att32b_decode", "sequences": Bn, "q_heads": Hq,
                       "kv_heads": Hkv, "head_dim": D, "page": page, "cached_tokens": tokens,
                       "step_algorithmic_bytes": work},
            "roofline": {"bound": "hbm", "kernel": dom,
                         "achieved": round(work / us[dom] / 1e3, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(work / us[dom] / 1e3 / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(dom, "att32b_decode")},
            "kernels": {k: {"us": round(v, 2), "algorithmic_bytes": work,
                            "GB/s": round(work / v / 1e3, 1)} for k, v in us.items()},
            "batch_sizes": tail}
    if not args.no_cpu_baseline:
        from oracle import attention as oatt
        from oracle import kv as okv
        rows = list(range(0, Bn, 8))                     # 8 of the 64 sequences
        t0 = time.perf_counter()
        oatt.decode_attention(q_np, okv.kv_scale(q_np), kc_np, vc_np, np.float32(2.0 ** -12),
                              np.float32(2.0 ** -8), table, lens, Hkv, page, batch_rows=rows)
        ct = time.perf_counter() - t0
        sample = 2 * int(lens[rows].sum()) * Hkv * D + 4 * len(rows) * Hq * D
        line["cpu_baseline"] = {"value": round(sample / ct / 1e9, 4), "unit": "GB/s",
                                "cores": cpu_threads(), "os_cpu_count": os.cpu_count(), "kind": "oracle", "seconds": round(ct, 2),
                                "sample": f"sequences {rows[0]}, {rows[1]}, ... {rows[-1]} "
                                          f"({len(rows)} of {Bn}) of the same batch"}
    return line


def run_tis(args, torch, B, W):
    """Rollout correction of a batch of 1024 responses padded to 8192 tokens:
    per step, the TIS and the MIS weights with per-sequence statistics and
    batch totals (two calls)."""
    cfg = W.TIS_BATCH
    Bn, T, cap = cfg["B"], cfg["T"], cfg["cap"]
    p = W.tis_batch(Bn, T, seed=0)
    lt = torch.from_numpy(p["lp_train"]).cuda()
    lr = torch.from_numpy(p["lp_rollout"]).cuda()
    mk = torch.from_numpy(p["mask"]).cuda()
    outs = {m: (torch.empty((Bn, T), dtype=torch.float32, device="cuda:0"),
                torch.empty((Bn, 4), dtype=torch.float32, device="cuda:0"),
                torch.empty((4,), dtype=torch.float64, device="cuda:0"))
            for m in (B.IS_TRUNCATE, B.IS_MASK)}
    names = {B.IS_TRUNCATE: "tis_token_weights(TIS)", B.IS_MASK: "tis_token_weights(MIS)"}

    def step(_i, timer=None):
        for m in (B.IS_TRUNCATE, B.IS_MASK):
            w, rs, tt = outs[m]
            f = lambda: B.tis_token_weights(lt, lr, mk, cap, m, out=w, row_stats=rs, totals=tt)
            timer.run(names[m], f) if timer else f()

    dt, us, dom = timed_steps(torch, step, args)
    per_call = 13 * Bn * T + 16 * Bn * 2 + 32          # inputs, weights, row stats (write + read), totals
    kernels = {k: {"us": round(v, 2), "algorithmic_bytes": per_call,
                   "GB/s": round(per_call / v / 1e3, 1)} for k, v in us.items()}
    line = {"metric": METRIC, "value": round(2 * per_call / dt / 1e9, 1), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(dt * 1e3, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "tis_batch", "sequences": Bn, "tokens": T, "cap": cap,
                       "valid_tokens": int(p["mask"].sum()),
                       "step": "TIS and MIS token weights with per-sequence statistics and totals"},
            "roofline": {"bound": "hbm", "kernel": dom,
                         "achieved": round(per_call / us[dom] / 1e3, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(per_call / us[dom] / 1e3 / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("tis_token_weights", "tis_batch")},
            "kernels": kernels}
    if not args.no_cpu_baseline:
        from oracle import tis as otis
        t0 = time.perf_counter()
        for m in (otis.TRUNCATE, otis.MASK):
            otis.importance_weights(p["lp_train"], p["lp_rollout"], p["mask"], cap, m)
        ct = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(2 * per_call / ct / 1e9, 4), "unit": "GB/s",
                                "cores": cpu_threads(), "os_cpu_count": os.cpu_count(), "kind": "oracle", "seconds": round(ct, 2),
                                "sample": "one whole step (TIS and MIS over the full batch)"}
    return line


def run_sync32b(args, torch, B, W):
    """Quantize-on-receive of the 32B-class up/gate weight (Wt [27648, 5120]
    bf16, 283 MB), the step that weight synchronization into the inference
    engine adds: the weight arrives in 8 chunks of 3456 rows (one tensor-
    parallel-8 shard each) from pinned host memory on a copy stream (the
    host link stands in for the link from the trainer), into two staging
    buffers in turn; each chunk is quantized into place in the full FP8
    weight (fp8_weight_block_quant_into) on the compute stream as soon as it
    has landed, while the next one is in transfer.  Reported: the step
    against the bare transfer of the same chunks and the bare quantization
    of resident chunks (all host-timed over whole steps)."""
    N, K, chunks = 27648, 5120, 8
    rows = N // chunks
    dev = torch.device("cuda:0")
    host_w = torch.empty((N, K), dtype=torch.int16, pin_memory=True)
    host_w.copy_(torch.from_numpy(W.weight(N, K, seed=0).view(np.int16)))
    stage = [torch.empty((rows, K), dtype=torch.int16, device=dev) for _ in range(2)]
    q = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sc = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    copy_stream = torch.cuda.Stream(device=dev)          # default priority
    comp = torch.cuda.current_stream(dev)
    landed = [torch.cuda.Event() for _ in range(chunks)]
    consumed = [torch.cuda.Event() for _ in range(chunks)]

    def sync_step(quantize=True, transfer=True):
        for c in range(chunks):
            buf = stage[c % 2]
            if transfer:
                with torch.cuda.stream(copy_stream):
                    if c >= 2:
                        copy_stream.wait_event(consumed[c - 2])
                    buf.copy_(host_w[c * rows:(c + 1) * rows], non_blocking=True)
                    landed[c].record(copy_stream)
                comp.wait_event(landed[c])
            if quantize:
                B.fp8_weight_block_quant_into(buf, q, sc, row0=c * rows)
            consumed[c].record(comp)

    def host_timed(f, n):
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            f()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    dt = host_timed(lambda: sync_step(), args.steps)
    dt_copy = host_timed(lambda: sync_step(quantize=False), args.steps)
    dt_quant = host_timed(lambda: sync_step(transfer=False), args.steps)
    torch.cuda.synchronize()
    # the step's result is the full weight's quantization
    ref_q, ref_s = B.fp8_weight_block_quant(torch.from_numpy(W.weight(N, K, seed=0).view(np.int16)).to(dev))
    sync_step()
    torch.cuda.synchronize()
    same = bool(torch.equal(q, ref_q) and torch.equal(sc, ref_s))
    wbytes = 2 * N * K
    qbytes = quant_bytes(N, K, (N // 128) * (K // 128))
    line = {"metric": METRIC, "value": round(wbytes / dt / 1e9, 1), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(dt * 1e3, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8e4m3", "data": "synthetic",
            "config": {"workload": "sync32b_requant", "N": N, "K": K, "chunks": chunks,
                       "source": "pinned host memory (stands in for the inter-GPU link)",
                       "value": "bf16 weight bytes received and quantized per second"},
            "transfer_only_ms": round(dt_copy * 1e3, 4),
            "quantize_only_ms": round(dt_quant * 1e3, 4),
            "overhead_vs_transfer": round(dt / dt_copy - 1.0, 4),
            "link_GB/s": round(wbytes / dt_copy / 1e9, 1),
            "same_as_whole_weight_quant": same,
            "roofline": {"bound": "hbm", "kernel": "fp8_weight_block_quant_into",
                         "achieved": round(qbytes / dt_quant / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(qbytes / dt_quant / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": None}}
    if not args.no_cpu_baseline:
        from oracle import quant as oq
        chunk = W.weight(N, K, seed=0)[:rows]
        t0 = time.perf_counter()
        oq.fp8_weight_block_quant(chunk)
        ct = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(2 * rows * K / ct / 1e9, 4), "unit": "GB/s",
                                "cores": cpu_threads(), "os_cpu_count": os.cpu_count(), "kind": "oracle", "seconds": round(ct, 2),
                                "sample": f"one chunk ({rows} x {K}) quantized by the oracle"}
    return line


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode7b_upgate",
                    choices=["decode7b_upgate", "decode32b_sweep", "prefill32b", "stack32b_requant",
                             "kv32b_prefill", "moe_decode", "tis_batch", "stack32b_gemm",
                             "att32b_decode", "sync32b_requant"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 512 MiB device copy three times (outside the "
                         "timed region): the reference kernel for scaling rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: this path is a single-GPU kernel library "
              "(a data-parallel deployment runs one independent copy per GPU); run with --gpus 1.",
              file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    from precision_rl_rollout_amd import binding as B
    from precision_rl_rollout_amd import workloads as W
    B.load()
    if args.copy_calibration:
        src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    run = {"decode7b_upgate": run_decode7b, "decode32b_sweep": run_decode32b,
           "prefill32b": run_prefill32b, "stack32b_requant": run_stack32b,
           "kv32b_prefill": run_kv32b, "moe_decode": run_moe_decode,
           "tis_batch": run_tis, "stack32b_gemm": run_stack_gemm,
           "att32b_decode": run_att, "sync32b_requant": run_sync32b}[args.workload]
    line = run(args, torch, B, W)
    if TIMINGS:
        line["timing"] = TIMINGS
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
