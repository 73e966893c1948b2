"""Regenerate the rocprofv3 summaries committed under profiles/ (GPU host only).

    python -m conv2d_batchnorm_silu_amd.make_profiles --raw gpurun_out/prof \
        [--traces] [--split] [--counters] [--util] [--workloads W1,W2]

* ``--traces``: one ``--kernel-trace --stats`` run of ``bench.py --only`` per
  workload -> ``profiles/kernel_trace_<workload>.txt`` (average duration of
  the fused kernel per launch, with its algorithmic GB/s and TFLOP/s).
* ``--split``: the same for the fused, split (conv kernel, then one
  BatchNorm+SiLU kernel) and unfused (conv, BatchNorm, SiLU) plans of every
  fp16 workload, with each kernel's registers and LDS from the trace ->
  ``profiles/fused_vs_split.md``.
* ``--counters``: ``FETCH_SIZE`` and ``WRITE_SIZE`` (each in its own
  ``--pmc`` run) of each workload's fused kernel and of a plain device copy
  of known size (``copy_calibration.py``), which gives the scale of each
  counter -> ``profiles/counters.json`` and
  ``profiles/hbm_traffic_<workload>.txt``.
* ``--util``: one ``--pmc`` run per workload with the matrix-core, LDS and
  VALU activity counters of its fused kernel (MFMA busy cycles against the
  GPU's active cycles times the SIMD count, MFMA FLOPs counted by the
  hardware against the algorithmic FLOPs, LDS instructions and bank-conflict
  cycles) -> ``profiles/util_<workload>.txt`` and ``counters.json``.

Raw rocprofv3 output stays under ``--raw``. Every profiled program is run as
``rocprofv3 ... -- python3 <script>`` from /tmp with TMPDIR=/tmp; this
process itself never touches the GPU.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")  # --dest overrides
REUSE = False  # --reuse: summarise raw output already under --raw, run nothing
sys.path.insert(0, ROOT)

from conv2d_batchnorm_silu_amd import profiling, traffic  # noqa: E402
from conv2d_batchnorm_silu_amd.inputs import HEADLINE, WORKLOADS  # noqa: E402

BENCH = os.path.join(ROOT, "bench.py")
COPY = os.path.join(PKG, "copy_calibration.py")


def log(msg):
    print("[make_profiles] " + msg, flush=True)


def run_profiled(raw, name, prof_args, prog_args, limit):
    """rocprofv3 <prof_args> -d raw/name -o run -- python3 <prog_args>; the
    whole command under `timeout -s KILL limit`. Returns the output dir.
    rocprofv3 may end with a signal after a complete run, so success is
    judged by the CSV it leaves."""
    out = os.path.join(raw, name)
    if REUSE:
        return out
    cmd = (["timeout", "-s", "KILL", str(limit), "rocprofv3"] + prof_args +
           ["-f", "csv", "-d", out, "-o", "run", "--", "python3"] + prog_args)
    env = dict(os.environ, TMPDIR="/tmp")
    log("run %s: %s" % (name, " ".join(cmd)))
    with open(os.path.join(raw, name + ".log"), "w") as f:
        rc = subprocess.run(cmd, cwd="/tmp", env=env, stdout=f, stderr=subprocess.STDOUT).returncode
    log("%s finished, status %d" % (name, rc))
    if rc in (124, 137) or rc == -9:
        raise RuntimeError("%s hit its time limit" % name)
    return out


def find_csv(out, suffix):
    hits = sorted(glob.glob(os.path.join(out, "**", "*" + suffix), recursive=True))
    if not hits:
        raise RuntimeError("no %s under %s" % (suffix, out))
    return hits[-1]


def cmd_text(prof_args, prog_args):
    rel = [a.replace(ROOT, "<repo>") for a in prog_args]
    return "cd /tmp && rocprofv3 %s -f csv -d <out> -o run -- python3 %s" % (
        " ".join(prof_args), " ".join(rel))


def fused_row(stats):
    """The fused conv kernel of a bench --only run: the most-called kernel
    whose name is one of this library's conv kernels."""
    rows = [r for r in stats if "conv2d_bn_silu" in r["name"]]
    return max(rows, key=lambda r: r["calls"])


TRACE_STEPS = 50  # timed steps of every profiled bench.py --only run


def write_trace(raw, wl):
    prof = ["--kernel-trace", "--stats", "-T"]
    prog = [BENCH, "--only", "--workload", wl.name, "--steps", str(TRACE_STEPS), "--warmup", "5"]
    out = run_profiled(raw, "trace_" + wl.name, prof, prog, 180)
    stats = profiling.kernel_stats(find_csv(out, "_kernel_stats.csv"))
    timed = profiling.timed_region(find_csv(out, "_kernel_trace.csv"), TRACE_STEPS)
    fb, fl = traffic.fused_bytes(wl), traffic.conv_flops(wl)
    lines = ["# rocprofv3 kernel-trace summary: fused conv2d+BN+SiLU, workload %s" % wl.name,
             "# shape: N=%d H=%d W=%d C_in=%d C_out=%d k=%dx%d s=%d p=%d (%s)" % (
                 wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad, wl.dtype),
             "# command: " + cmd_text(prof, prog),
             "# algorithmic bytes per launch %d, conv FLOP per launch %d" % (fb, fl),
             "# all dispatches of the run (clock-settling phase, warmup and timed steps):",
             "# kernel | calls | avg us | min us | max us | % of GPU time | "
             "GB/s (algorithmic, avg) | TFLOP/s (avg)"]
    fr = fused_row(stats)
    for r in stats:
        cells = [r["name"][:110], str(r["calls"]), "%.2f" % (r["avg_ns"] / 1e3),
                 "%.2f" % (r["min_ns"] / 1e3), "%.2f" % (r["max_ns"] / 1e3), "%.1f" % r["pct"]]
        if r is fr:
            cells += ["%.1f" % (fb / r["avg_ns"]), "%.2f" % (fl / r["avg_ns"] / 1e3)]
        lines.append(" | ".join(cells))
    t = timed[fr["name"]]
    lines += ["# timed region (the fused kernel's last %d dispatches = bench.py's timed steps):"
              % t["n"],
              "# avg duration %.2f us (%.1f GB/s algorithmic, %.2f TFLOP/s), start-to-start "
              "%.2f us per step" % (t["avg_ns"] / 1e3, fb / t["avg_ns"], fl / t["avg_ns"] / 1e3,
                                    t["spacing_ns"] / 1e3)]
    path = os.path.join(PROFILES, "kernel_trace_%s.txt" % wl.name)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    log("wrote " + path)
    TRACE_NS[wl.name] = t["avg_ns"]
    return fr


TRACE_NS = {}  # workload -> timed-region average duration of its fused kernel (ns)


def trace_ns(wl):
    """The fused kernel's duration from this run's trace, else from the
    kernel-trace summary under profiles/."""
    if wl.name in TRACE_NS:
        return TRACE_NS[wl.name]
    try:
        with open(os.path.join(PROFILES, "kernel_trace_%s.txt" % wl.name)) as f:
            for line in f:
                if line.startswith("# avg duration "):
                    return float(line.split()[3]) * 1e3
    except OSError:
        pass
    return None


def compiler_resources():
    """Kernel symbol -> dict of VGPRs, AGPRs, SGPRs, spills, static LDS and
    scratch bytes, from the code-object metadata of each source compiled to
    gfx950 assembly with the library's own flags (host-side: hipcc only)."""
    import concurrent.futures as cf
    import re
    import tempfile
    from conv2d_batchnorm_silu_amd import build as Bld

    def one(src):
        with tempfile.TemporaryDirectory(prefix="tg_res_") as d:
            out = os.path.join(d, "k.s")
            r = subprocess.run([Bld.hipcc()] + Bld.HIPCC_FLAGS +
                               ["--cuda-device-only", "-S", src, "-o", out],
                               capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError("hipcc failed for %s" % src)
            return open(out).read()

    res = {}
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        for asm in ex.map(one, Bld.sources()):
            meta = asm[asm.find("amdhsa.kernels:"):]
            for blk in re.split(r"\n  - ", meta)[1:]:
                kv = dict(re.findall(r"\.([a-z_]+):\s+(\S+)", blk))
                if "name" not in kv:
                    continue
                res[kv["name"]] = {k: kv.get(k, "n/a") for k in (
                    "vgpr_count", "agpr_count", "sgpr_count", "vgpr_spill_count",
                    "sgpr_spill_count", "group_segment_fixed_size",
                    "private_segment_fixed_size")}
    return res


def lookup(res, name):
    for sym, v in res.items():
        if sym.startswith(name) or name.startswith(sym):
            return v
    return None


def write_split(raw, names):
    prof = ["--kernel-trace", "--stats", "-T"]
    res = compiler_resources()
    lines = ["# Fused vs split vs unfused, per workload (one MI355X)",
             "",
             "Split = the conv kernel with an identity epilogue writing t1 (fp16), then one "
             "BatchNorm+SiLU streaming kernel; unfused = conv, BatchNorm, SiLU as three kernels. "
             "Durations are rocprofv3 kernel-trace averages per launch (kernel time only, no "
             "launch gaps) over the timed steps (each kernel's last %d dispatches; the earlier "
             "ones are bench.py's clock-settling and warmup calls); the sum over a plan's "
             "kernels is its GPU time per step. Registers, "
             "spills, static LDS and scratch come from the code-object metadata of the "
             "library's gfx950 build (dynamic LDS is requested per launch by the plan and is "
             "not included); VGPR+AGPR sets the waves a SIMD can hold (512 registers per "
             "lane: 2 waves at 256, 3 at 168, 4 at 128)." % TRACE_STEPS,
             "",
             "command per workload W and plan K: " +
             cmd_text(prof, [BENCH, "--only", "--workload", "W", "--plan", "K", "--steps",
                             str(TRACE_STEPS), "--warmup", "5"]),
             ""]
    for name in names:
        wl = WORKLOADS[name]
        lines += ["## %s (%s)" % (name, "N=%d %dx%d C_in=%d -> C_out=%d, %dx%d s%d p%d" % (
            wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad)), "",
                  "plan | kernel | calls | avg us | VGPR | AGPR | SGPR | spills (V/S) | "
                  "static LDS B | scratch B",
                  "---|---|---|---|---|---|---|---|---|---"]
        totals = {}
        for kind in ("auto", "split", "unfused"):
            prog = [BENCH, "--only", "--workload", name, "--plan", kind, "--steps",
                    str(TRACE_STEPS), "--warmup", "5"]
            out = run_profiled(raw, "split_%s_%s" % (name, kind), prof, prog, 180)
            stats = profiling.kernel_stats(find_csv(out, "_kernel_stats.csv"))
            timed = profiling.timed_region(find_csv(out, "_kernel_trace.csv"), TRACE_STEPS)
            calls = max(r["calls"] for r in stats if "conv2d_bn_silu" in r["name"])
            tot = 0.0
            for r in stats:
                # the plan's own kernels: launched once per step
                if r["calls"] != calls:
                    continue
                v = lookup(res, r["name"]) or {}
                g = lambda k: v.get(k, "n/a")
                lines.append("%s | %s | %d | %.2f | %s | %s | %s | %s/%s | %s | %s" % (
                    "fused" if kind == "auto" else kind, r["name"][:90], r["calls"],
                    timed[r["name"]]["avg_ns"] / 1e3, g("vgpr_count"), g("agpr_count"), g("sgpr_count"),
                    g("vgpr_spill_count"), g("sgpr_spill_count"),
                    g("group_segment_fixed_size"), g("private_segment_fixed_size")))
                tot += timed[r["name"]]["avg_ns"] / 1e3
            totals[kind] = tot
        lines += ["", "GPU time per step: fused %.2f us, split %.2f us (%.2fx), unfused %.2f us "
                  "(%.2fx)" % (totals["auto"], totals["split"], totals["split"] / totals["auto"],
                               totals["unfused"], totals["unfused"] / totals["auto"]), ""]
    path = os.path.join(PROFILES, "fused_vs_split.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    log("wrote " + path)


_COPY_KIB = {}  # (counter, mode) -> KiB per dispatch of the calibration copy (one run each)
CALIBRATIONS = (("", []), ("_dma", ["--dma"]), ("_rotate", ["--rotate"]))  # first: the one used


def copy_kib(raw, counter, mode=""):
    """The counter's value per dispatch for a copy of COPY_BYTES: torch's
    copy of one buffer pair (mode ""), this library's copy that reads through
    direct-to-LDS buffer loads ("_dma"), or torch's copy over four buffer
    pairs ("_rotate")."""
    key = (counter, mode)
    if key not in _COPY_KIB:
        name = "pmc_%s_copy%s" % (counter.lower(), mode)
        cout = run_profiled(raw, name, ["--pmc", counter], [COPY] + dict(CALIBRATIONS)[mode], 60)
        cpath = find_csv(cout, "_counter_collection.csv")
        cv, cn = profiling.counter_per_dispatch(cpath, "copy", counter)
        if cv is None:  # the copy kernel's name varies between torch builds
            cv, cn = profiling.counter_per_dispatch(cpath, "", counter)
        _COPY_KIB[key] = cv
    return _COPY_KIB[key]


def fused_symbol(path):
    """The most dispatched conv2d_bn_silu kernel of a counter or trace CSV."""
    with open(path) as f:
        names = collections.Counter(r["Kernel_Name"] for r in csv.DictReader(f)
                                    if "conv2d_bn_silu" in r["Kernel_Name"])
    return names.most_common(1)[0][0]


def write_counters(raw, wl, source_hash):
    prog = [BENCH, "--only", "--workload", wl.name, "--steps", "20", "--warmup", "2"]
    val = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        out = run_profiled(raw, "pmc_%s_%s" % (counter.lower(), wl.name), ["--pmc", counter],
                           prog, 60)
        path = find_csv(out, "_counter_collection.csv")
        sym = fused_symbol(path)
        v, n = profiling.counter_per_dispatch(path, sym, counter)
        from conv2d_batchnorm_silu_amd.copy_calibration import COPY_BYTES
        scales = {m: COPY_BYTES / (copy_kib(raw, counter, m) * 1024.0) for m, _ in CALIBRATIONS}
        val[counter] = dict(raw_kib=v, dispatches=n, copy_kib=copy_kib(raw, counter),
                            symbol=sym, copy_scales=scales)
    # Scales. The copies' absolute scales vary between runs and buffer
    # reuse (recorded below), but in every copy FETCH_SIZE's scale is the
    # same multiple of WRITE_SIZE's, and this kernel writes y exactly once:
    # WRITE_SIZE is scaled to y's bytes, FETCH_SIZE by the copy's ratio.
    b = traffic.workload_bytes(wl)
    wscale = b["y"] / (val["WRITE_SIZE"]["raw_kib"] * 1024.0)
    ratio = val["FETCH_SIZE"]["copy_scales"][""] / val["WRITE_SIZE"]["copy_scales"][""]
    for counter, sc in (("FETCH_SIZE", wscale * ratio), ("WRITE_SIZE", wscale)):
        val[counter]["scale"] = sc
        val[counter]["bytes"] = val[counter]["raw_kib"] * 1024.0 * sc
    alg = traffic.fused_bytes(wl)
    hbm = val["FETCH_SIZE"]["bytes"] + val["WRITE_SIZE"]["bytes"]
    sym = val["FETCH_SIZE"]["symbol"]
    entry = {"source_hash": source_hash, "kernel_symbol": sym,
             "fetch_kib_raw": val["FETCH_SIZE"]["raw_kib"],
             "write_kib_raw": val["WRITE_SIZE"]["raw_kib"],
             "fetch_scale": val["FETCH_SIZE"]["scale"], "write_scale": val["WRITE_SIZE"]["scale"],
             "copy_scales": {c: val[c]["copy_scales"] for c in ("FETCH_SIZE", "WRITE_SIZE")},
             "fetch_over_write_scale_of_copy": ratio,
             "fetch_bytes": val["FETCH_SIZE"]["bytes"], "write_bytes": val["WRITE_SIZE"]["bytes"],
             "hbm_bytes_per_launch": int(round(hbm)), "algorithmic_bytes": alg,
             "excess_frac": hbm / alg - 1.0}
    cpath = os.path.join(PROFILES, "counters.json")
    try:
        with open(cpath) as f:
            allc = json.load(f)
    except (OSError, ValueError):
        allc = {}
    allc[wl.name] = entry
    with open(cpath, "w") as f:
        json.dump(allc, f, indent=1)
    lines = ["# HBM traffic of the fused kernel, workload %s (N=%d %dx%d C_in=%d -> C_out=%d, "
             "%dx%d, %s)" % (wl.name, wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.dtype),
             "# commands (cd /tmp; TMPDIR=/tmp), each counter in its own run:"]
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        lines.append("#   " + cmd_text(["--pmc", counter], prog))
    cs = lambda c, m: val[c]["copy_scales"][m]
    lines += ["# calibration: a %d MiB device copy (reads and writes exactly %d bytes), each "
              "counter in its own run, three ways: torch's copy of one buffer pair, this "
              "library's copy reading through direct-to-LDS loads, torch's copy over four "
              "buffer pairs:" % (COPY_BYTES_MIB(), COPY_BYTES_MIB() * 2**20),
              "#   " + cmd_text(["--pmc", "FETCH_SIZE"], [COPY]) + "   (and WRITE_SIZE; "
              "and with --dma, --rotate)",
              "# copy scales FETCH / WRITE: one pair %.4f / %.4f, direct-to-LDS %.4f / %.4f, four "
              "pairs %.4f / %.4f (the absolute scale moves with the run and with buffer reuse; "
              "the ratio stays %.3f)" % (cs("FETCH_SIZE", ""), cs("WRITE_SIZE", ""),
                                        cs("FETCH_SIZE", "_dma"), cs("WRITE_SIZE", "_dma"),
                                        cs("FETCH_SIZE", "_rotate"), cs("WRITE_SIZE", "_rotate"),
                                        ratio),
              "# applied: WRITE_SIZE scaled to y's bytes (written exactly once; raw x 1024 / y = "
              "%.4f), FETCH_SIZE by that scale times the copy ratio: %.4f / %.4f" % (
                  1.0 / wscale, val["FETCH_SIZE"]["scale"], val["WRITE_SIZE"]["scale"]),
              "kernel %s (source hash %s), %d dispatches averaged" % (
                  sym[:80], source_hash, val["FETCH_SIZE"]["dispatches"]),
              "FETCH_SIZE raw %.1f KiB -> %.3f MB   (algorithmic reads x+w+BN = %.3f MB)" % (
                  val["FETCH_SIZE"]["raw_kib"], val["FETCH_SIZE"]["bytes"] / 1e6,
                  (b["x"] + b["w"] + b["bn"]) / 1e6),
              "WRITE_SIZE raw %.1f KiB -> %.3f MB   (algorithmic writes y = %.3f MB)" % (
                  val["WRITE_SIZE"]["raw_kib"], val["WRITE_SIZE"]["bytes"] / 1e6, b["y"] / 1e6),
              "total %.3f MB vs algorithmic %.3f MB -> excess %+.2f%%" % (
                  hbm / 1e6, alg / 1e6, 100.0 * (hbm / alg - 1.0))]
    path = os.path.join(PROFILES, "hbm_traffic_%s.txt" % wl.name)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    log("wrote %s and %s" % (path, cpath))


UTIL_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_BUSY_CYCLES",
                 "SQ_INSTS_LDS", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT",
                 "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE")
SIMDS = 1024  # 256 CUs x 4
CLOCK_GHZ = 2.4
MFMA_F16_PEAK_TFLOPS = 2516.6  # published dense fp16 MFMA peak


def per_dispatch_max(path, sym, counter):
    """Average over dispatches of the largest instance value (GRBM counters
    repeat the GPU-wide value per instance)."""
    per = collections.defaultdict(float)
    with open(path) as f:
        for r in csv.DictReader(f):
            if sym in r["Kernel_Name"] and r["Counter_Name"] == counter:
                per[r["Dispatch_Id"]] = max(per[r["Dispatch_Id"]], float(r["Counter_Value"]))
    return (sum(per.values()) / len(per), len(per)) if per else (None, 0)


def write_util(raw, wl, source_hash):
    prog = [BENCH, "--only", "--workload", wl.name, "--steps", "20", "--warmup", "2"]
    args = ["--pmc"] + list(UTIL_COUNTERS)
    out = run_profiled(raw, "util_%s" % wl.name, args, prog, 60)
    path = find_csv(out, "_counter_collection.csv")
    sym = fused_symbol(path)
    v = {}
    for c in UTIL_COUNTERS:
        if c.startswith("GRBM_"):
            v[c], n = per_dispatch_max(path, sym, c)
        else:
            v[c], n = profiling.counter_per_dispatch(path, sym, c)
    dur_ns = trace_ns(wl)
    clk = dur_ns * CLOCK_GHZ if dur_ns else None  # kernel clocks at the peak engine clock
    mfma_flop = v["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512
    alg_flop = traffic.conv_flops(wl)
    entry = {
        "source_hash": source_hash, "kernel_symbol": sym, "dispatches": n, "raw": v,
        "kernel_us": dur_ns / 1e3 if dur_ns else None,
        "mfma_busy_frac": v["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * clk) if clk else None,
        "mfma_flop_frac_of_peak": (mfma_flop / dur_ns / 1e3 / MFMA_F16_PEAK_TFLOPS
                                   if dur_ns else None),
        "mfma_flop_counted": mfma_flop, "algorithmic_flop": alg_flop,
        "mfma_flop_over_algorithmic": mfma_flop / alg_flop if alg_flop else None,
        "lds_bank_conflict_frac": (v["SQ_LDS_BANK_CONFLICT"] / v["SQ_ACTIVE_INST_LDS"]
                                   if v["SQ_ACTIVE_INST_LDS"] else None),
        "valu_active_per_inst": (v["SQ_ACTIVE_INST_VALU"] / v["SQ_INSTS_VALU"]
                                 if v["SQ_INSTS_VALU"] else None),
    }
    cpath = os.path.join(PROFILES, "counters.json")
    try:
        with open(cpath) as f:
            allc = json.load(f)
    except (OSError, ValueError):
        allc = {}
    allc.setdefault(wl.name, {})["util"] = entry
    with open(cpath, "w") as f:
        json.dump(allc, f, indent=1)
    fmt = lambda x: "n/a" if x is None else "%.4g" % x
    lines = ["# Matrix-core, LDS and VALU activity of the fused kernel, workload %s (N=%d %dx%d "
             "C_in=%d -> C_out=%d, %dx%d, %s)" % (wl.name, wl.N, wl.H, wl.W, wl.C_in, wl.C_out,
                                                   wl.kh, wl.kw, wl.dtype),
             "# command (cd /tmp; TMPDIR=/tmp; one pass, 8 SQ counters and 1 GRBM counter):",
             "#   " + cmd_text(args, prog),
             "kernel %s (source hash %s), %d dispatches averaged" % (sym[:80], source_hash, n)]
    for c in UTIL_COUNTERS:
        lines.append("%-30s %.6g per dispatch" % (c, v[c]))
    lines += [
        "fused kernel duration (timed region of its kernel trace) %s us" % fmt(entry["kernel_us"]),
        "MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES (summed over the %d SIMDs) / (%d x duration x "
        "%.1f GHz) = %s" % (SIMDS, SIMDS, CLOCK_GHZ, fmt(entry["mfma_busy_frac"])),
        "MFMA rate: counted MFMA FLOPs / duration / %.1f TFLOP/s (dense fp16 peak) = %s" % (
            MFMA_F16_PEAK_TFLOPS, fmt(entry["mfma_flop_frac_of_peak"])),
        "MFMA FLOPs counted (SQ_INSTS_VALU_MFMA_MOPS_F16 x 512) = %.4g vs algorithmic %.4g "
        "(ratio %s: padding and tail blocks the matrix cores still compute)" % (
            mfma_flop, alg_flop, fmt(entry["mfma_flop_over_algorithmic"])),
        "LDS: SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS = %s (bank-conflict stall cycles per "
        "LDS-issue cycle)" % fmt(entry["lds_bank_conflict_frac"]),
        "VALU active cycles per VALU instruction (SQ_ACTIVE_INST_VALU / SQ_INSTS_VALU) = %s" %
        fmt(entry["valu_active_per_inst"])]
    path_txt = os.path.join(PROFILES, "util_%s.txt" % wl.name)
    with open(path_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    log("wrote %s" % path_txt)


def COPY_BYTES_MIB():
    from conv2d_batchnorm_silu_amd.copy_calibration import COPY_BYTES
    return COPY_BYTES // 2**20


def _cold(q):
    return "%s (%s-%s)" % (q["p50"], q["p10"], q["p90"]) if q else None


def write_bench_table(path_json):
    """profiles/bench_per_workload.md from the JSON line of a default
    `python bench.py` run."""
    with open(path_json) as f:
        r = json.loads(f.read().strip().splitlines()[-1])
    lines = ["# bench.py per-workload results on one MI355X (fused kernel chosen by the MI355X "
             "dispatch table)",
             "# command: python bench.py   (defaults: --steps %d --warmup %d, settle %s ms; %s "
             "rotating input/output sets per workload)" % (
                 r["steps"], r["warmup"], r.get("settle_ms"),
                 r["config"].get("buffer_sets", "?")),
             "# times: HIP events over the timed steps on the launch stream, divided by the step "
             "count (includes launch gaps); timed calls go straight to the C ABI",
             "# split = conv kernel + one BatchNorm+SiLU kernel; unfused = conv, BatchNorm, SiLU; "
             "nchw legs = x NCHW->NHWC + fused + y NHWC->NCHW; train = batch-statistics "
             "BatchNorm (1x1 and stems: statistics-only conv, fold, fused conv; others: conv, statistics, "
             "fold, BatchNorm+SiLU); packed = the fused kernel "
             "reading a filter packed once at load time into its tile order",
             "# cold = a 1 GiB cache flush before every single call, events around that call "
             "(p50, with p10-p90); predicted x = (fused + 2 launches + 4|y| at the measured "
             "device-copy bandwidth) / fused",
             "workload | kernel | us | TFLOP/s | GB/s (algorithmic) | bound | frac of bound peak "
             "| unfused us | x vs unfused | split us | x vs split | relu / gelu / none us | "
             "nchw legs us (share) | train us | fp8 y us (GB/s) | + residual us (GB/s) | "
             "packed us | cold us p50 (p10-p90) | unfused cold us p50 | x vs unfused cold | "
             "predicted x"]
    for c in r["per_config"]:
        a = c.get("act_us", {})
        lines.append(" | ".join(str(v) for v in [
            c["workload"], c["kernel"].split(" f16 ")[0].split(" f32 ")[0], c["us"], c["tflops"],
            c["gbs"], c["bound"], c["frac"], c.get("unfused_us"), c.get("speedup_vs_unfused"),
            c.get("split_us"), c.get("speedup_vs_split"),
            "%s / %s / %s" % (a.get("relu"), a.get("gelu"), a.get("none")),
            "%s (%s)" % (c.get("nchw_legs_us"), c.get("nchw_legs_share")), c.get("train_us"),
            "%s (%s)" % (c.get("fp8_out_us"), c.get("fp8_out_gbs")),
            "%s (%s)" % (c.get("residual_us"), c.get("residual_gbs")), c.get("packed_us"),
            _cold(c.get("cold_us")), (c.get("unfused_cold_us") or {}).get("p50"),
            c.get("speedup_vs_unfused_cold"), c.get("predicted_speedup_vs_unfused")]))
    if r.get("cpu_baseline"):
        lines.append("cpu_baseline (fp64 oracle, headline workload): " +
                     json.dumps(r["cpu_baseline"]))
    lines.append("roofline (headline): " + json.dumps(r["roofline"]))
    if r.get("frac_of_copy") is not None:
        lines.append("headline against the measured device-copy rate (%s GB/s): %s" % (
            r["per_config"][[c["workload"] for c in r["per_config"]].index(
                r["config"]["workload"])].get("copy_gbs"), r["frac_of_copy"]))
    if r.get("device"):
        lines.append("device: " + json.dumps(r["device"]))
    lines.append("value: %s %s (%s)" % (r["value"], r["unit"], r["config"]["workload"]))
    path = os.path.join(PROFILES, "bench_per_workload.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    log("wrote " + path)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--raw", required=True, help="directory for raw rocprofv3 output")
    ap.add_argument("--traces", action="store_true")
    ap.add_argument("--split", action="store_true")
    ap.add_argument("--counters", action="store_true")
    ap.add_argument("--util", action="store_true")
    ap.add_argument("--workloads", default=None, help="comma-separated (default: all)")
    ap.add_argument("--dest", default=None, help="where the summaries go (default: profiles/)")
    ap.add_argument("--bench-json", default=None,
                    help="format the JSON line of a bench.py run into bench_per_workload.md")
    ap.add_argument("--reuse", action="store_true",
                    help="summarise the raw output already under --raw without profiling")
    args = ap.parse_args()
    global PROFILES, REUSE
    if args.dest:
        PROFILES = os.path.abspath(args.dest)
        os.makedirs(PROFILES, exist_ok=True)
    REUSE = args.reuse
    raw = os.path.abspath(args.raw)
    os.makedirs(raw, exist_ok=True)
    names = args.workloads.split(",") if args.workloads else [
        n for n, w in WORKLOADS.items() if w.dtype == "f16"]
    import bench  # source_hash only; bench imports torch lazily
    if args.traces:
        for n in names:
            write_trace(raw, WORKLOADS[n])
    if args.split:
        write_split(raw, names)
    if args.counters:
        for n in names:
            write_counters(raw, WORKLOADS[n], bench.source_hash())
    if args.util:
        for n in names:
            write_util(raw, WORKLOADS[n], bench.source_hash())
    if args.bench_json:
        write_bench_table(args.bench_json)


if __name__ == "__main__":
    main()
