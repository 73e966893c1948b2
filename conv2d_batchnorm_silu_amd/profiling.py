"""Summaries of rocprofv3 output for the measurement reports.

* ``kernel_stats(csv)``: per-kernel calls / average / total duration from a
  ``--kernel-trace --stats`` run (``*_kernel_stats.csv``).
* ``counter_per_dispatch(csv, name_substr, counter)``: the average value of
  one PMC counter (summed over its hardware instances) per dispatch of the
  kernels whose name contains ``name_substr`` (``--pmc`` run,
  ``*_counter_collection.csv``).
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
