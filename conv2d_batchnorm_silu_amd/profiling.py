"""Summaries of rocprofv3 output for the measurement reports.

* ``kernel_stats(csv)``: per-kernel calls / average / total duration from a
  ``--kernel-trace --stats`` run (``*_kernel_stats.csv``).
* ``counter_per_dispatch(csv, name_substr, counter)``: the average value of
  one PMC counter (summed over its hardware instances) per dispatch of the
  kernels whose name contains ``name_substr`` (``--pmc`` run,
  ``*_counter_collection.csv``).
* ``timed_region(csv, steps)``: per kernel, the average duration and the
  start-to-start spacing of its last ``steps`` dispatches
  (``*_kernel_trace.csv``). bench.py repeats every timed call untimed for a
  clock-settling phase and warmup before its timed steps, so in a
  ``bench.py --only --steps K`` run the last K dispatches of each of the
  plan's kernels are the timed steps.
FETCH_SIZE and WRITE_SIZE are reported by rocprofv3 in KiB per dispatch.
"""
from __future__ import annotations

import collections
import csv


def kernel_stats(path: str) -> list:
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({"name": r["Name"], "calls": int(r["Calls"]),
                         "avg_ns": float(r["AverageNs"]), "total_ns": float(r["TotalDurationNs"]),
                         "pct": float(r["Percentage"]), "min_ns": float(r["MinNs"]),
                         "max_ns": float(r["MaxNs"])})
    return rows


def timed_region(path: str, steps: int) -> dict:
    """Kernel name -> {"avg_ns", "spacing_ns", "n"} over its last `steps`
    dispatches (kernels dispatched fewer times are left out)."""
    per = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            per[r["Kernel_Name"]].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    out = {}
    for name, ds in per.items():
        if len(ds) < steps or steps < 2:
            continue
        ds = sorted(ds)[-steps:]
        out[name] = {"avg_ns": sum(e - s for s, e in ds) / steps,
                     "spacing_ns": (ds[-1][0] - ds[0][0]) / (steps - 1), "n": steps}
    return out


def counter_per_dispatch(path: str, name_substr: str, counter: str) -> tuple:
    """(average value per dispatch, number of dispatches)."""
    per = collections.defaultdict(float)
    with open(path) as f:
        for r in csv.DictReader(f):
            if name_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        return None, 0
    return sum(per.values()) / len(per), len(per)
