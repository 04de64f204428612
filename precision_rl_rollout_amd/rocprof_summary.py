"""Summaries of rocprofv3 output as the markdown tables kept under profiles/.

    python -m precision_rl_rollout_amd.rocprof_summary trace DIR [SPLIT]
    python -m precision_rl_rollout_amd.rocprof_summary counters DIR COUNTER [SPLIT]

``trace``: per-dispatch durations from DIR's ``*kernel_trace.csv`` grouped
by kernel, grid (workgroups), LDS allocation and register count, with the
call count and mean / min / max microseconds.

``counters``: the mean of COUNTER (e.g. FETCH_SIZE, WRITE_SIZE, in KiB) per
dispatch from DIR's ``*counter_collection.csv``, grouped the same way.  When
the run included bench.py's ``--copy-calibration`` (a 512 MiB device copy,
256 workgroups), the copy's own reading gives the scale from counter units
to bytes moved (524288 KiB each way), printed first.

``SPLIT`` (``kernel=n1,n2,...``) cuts the dispatches of one launch shape of
that kernel, in dispatch order, into consecutive groups of n1, n2, ...
dispatches, reported as rows of their own (labelled ``#1``, ``#2``, ...;
dispatches past the listed counts form a last group): one kernel used in
several phases of a run (warm-up, timed steps, a second workload) shows per
phase.
"""

from __future__ import annotations

import collections
import csv
import glob
import os
import re
import statistics
import sys

COPY_KIB = 524288.0           # the calibration copy moves 512 MiB each way


def _one(directory: str, suffix: str) -> str:
    files = glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    return files[0]


def short_name(name: str) -> str:
    n = re.sub(r"<.*", "", name.split("(")[0].replace("void ", ""))
    return n.split("::")[-1]


def _key(row: dict) -> tuple:
    grid = int(row.get("Grid_Size_X", row.get("Grid_Size", 0)))
    wg = max(1, int(row.get("Workgroup_Size_X", row.get("Workgroup_Size", 1))))
    return (short_name(row["Kernel_Name"]), grid // wg, row.get("LDS_Block_Size", ""),
            row.get("Arch_VGPR_Count", row.get("VGPR_Count", "")))


def _order(row: dict) -> int:
    for k in ("Dispatch_Id", "Start_Timestamp", "Correlation_Id"):
        if row.get(k, "") not in ("", None):
            return int(row[k])
    return 0


def _split_groups(items: list, split: str | None) -> list:
    """[(key, value, order)] -> [(key, [values])] in first-seen key order,
    with SPLIT's kernel cut into consecutive dispatch groups."""
    kernel, sizes = None, []
    if split:
        kernel, counts = split.split("=", 1)
        sizes = [int(c) for c in counts.split(",") if c]
    groups: dict = collections.OrderedDict()
    for key, value, order in items:
        groups.setdefault(key, []).append((order, value))
    out = []
    for key, vals in groups.items():
        if kernel is None or key[0] != kernel:
            out.append((key, [v for _, v in vals]))
            continue
        vals.sort()
        start = 0
        for i, n in enumerate(sizes + [len(vals)]):
            part = vals[start:start + n]
            start += len(part)
            if part:
                out.append(((f"{key[0]} #{i + 1}",) + key[1:], [v for _, v in part]))
    return out


def trace_table(directory: str, split: str | None = None) -> str:
    items = []
    with open(_one(directory, "kernel_trace.csv")) as f:
        for row in csv.DictReader(f):
            us = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            items.append((_key(row), us, _order(row)))
    groups = _split_groups(items, split)
    lines = ["| kernel | workgroups | LDS bytes | VGPRs | calls | avg us | min us | max us |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for (name, wgs, lds, vgpr), v in groups:
        lines.append(f"| `{name}` | {wgs} | {lds} | {vgpr} | {len(v)} | "
                     f"{statistics.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(lines)


def counter_table(directory: str, counter: str, split: str | None = None) -> str:
    items = []
    with open(_one(directory, "counter_collection.csv")) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                items.append((_key(row), float(row["Counter_Value"]), _order(row)))
    groups = _split_groups(items, split)
    lines = []
    # FETCH_SIZE / WRITE_SIZE are in KiB; other counters (cycles, the
    # percent of a derived metric such as MfmaUtil) carry their own unit.
    kib = counter in ("FETCH_SIZE", "WRITE_SIZE")
    for (name, wgs, _lds, _vgpr), v in groups:
        if kib and name == "__amd_rocclr_copyBuffer" and wgs == 256:
            lines.append(f"calibration copy: {statistics.mean(v):.1f} KiB -> scale "
                         f"{COPY_KIB / statistics.mean(v):.4f}")
    unit = " KiB" if kib else ""
    lines += [f"| kernel | workgroups | LDS bytes | VGPRs | dispatches | {counter}{unit} (mean) |",
              "|---|---:|---:|---:|---:|---:|"]
    for (name, wgs, lds, vgpr), v in groups:
        lines.append(f"| `{name}` | {wgs} | {lds} | {vgpr} | {len(v)} | {statistics.mean(v):.1f} |")
    return "\n".join(lines)


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    if len(argv) >= 2 and argv[0] == "trace":
        print(trace_table(argv[1], argv[2] if len(argv) > 2 else None))
        return 0
    if len(argv) >= 3 and argv[0] == "counters":
        print(counter_table(argv[1], argv[2], argv[3] if len(argv) > 3 else None))
        return 0
    print(__doc__, file=sys.stderr)
    return 2


if __name__ == "__main__":
    sys.exit(main())
