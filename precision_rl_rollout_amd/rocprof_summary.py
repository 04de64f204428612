"""Summaries of rocprofv3 output as the markdown tables kept under profiles/.

    python -m precision_rl_rollout_amd.rocprof_summary trace DIR
    python -m precision_rl_rollout_amd.rocprof_summary counters DIR COUNTER

``trace``: per-dispatch durations from DIR's ``*kernel_trace.csv`` grouped
by kernel, grid (workgroups), LDS allocation and register count, with the
call count and mean / min / max microseconds.

``counters``: the mean of COUNTER (e.g. FETCH_SIZE, WRITE_SIZE, in KiB) per
dispatch from DIR's ``*counter_collection.csv``, grouped the same way.  When
the run included bench.py's ``--copy-calibration`` (a 512 MiB device copy,
256 workgroups), the copy's own reading gives the scale from counter units
to bytes moved (524288 KiB each way), printed first.
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


def trace_table(directory: str) -> str:
    groups: dict = collections.OrderedDict()
    with open(_one(directory, "kernel_trace.csv")) as f:
        for row in csv.DictReader(f):
            us = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            groups.setdefault(_key(row), []).append(us)
    lines = ["| kernel | workgroups | LDS bytes | VGPRs | calls | avg us | min us | max us |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for (name, wgs, lds, vgpr), v in groups.items():
        lines.append(f"| `{name}` | {wgs} | {lds} | {vgpr} | {len(v)} | "
                     f"{statistics.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(lines)


def counter_table(directory: str, counter: str) -> str:
    groups: dict = collections.OrderedDict()
    with open(_one(directory, "counter_collection.csv")) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                groups.setdefault(_key(row), []).append(float(row["Counter_Value"]))
    lines = []
    for (name, wgs, _lds, _vgpr), v in groups.items():
        if name == "__amd_rocclr_copyBuffer" and wgs == 256:
            lines.append(f"calibration copy: {statistics.mean(v):.1f} KiB -> scale "
                         f"{COPY_KIB / statistics.mean(v):.4f}")
    lines += [f"| kernel | workgroups | LDS bytes | VGPRs | dispatches | {counter} KiB (mean) |",
              "|---|---:|---:|---:|---:|---:|"]
    for (name, wgs, lds, vgpr), v in groups.items():
        lines.append(f"| `{name}` | {wgs} | {lds} | {vgpr} | {len(v)} | {statistics.mean(v):.1f} |")
    return "\n".join(lines)


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    if len(argv) >= 2 and argv[0] == "trace":
        print(trace_table(argv[1]))
        return 0
    if len(argv) >= 3 and argv[0] == "counters":
        print(counter_table(argv[1], argv[2]))
        return 0
    print(__doc__, file=sys.stderr)
    return 2


if __name__ == "__main__":
    sys.exit(main())
