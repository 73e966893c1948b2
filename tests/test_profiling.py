"""CPU tests of the measurement helpers that summarise GPU runs:

  * profiling.timed_region: per kernel, the average duration and the
    start-to-start spacing of its last K dispatches (bench.py's timed steps
    follow its clock-settling and warmup calls), from a kernel-trace CSV;
  * make_profiles.write_bench_table: the per-workload table from a bench.py
    JSON line, including rows without the optional legs (None cells).
"""
import csv
import json

from conv2d_batchnorm_silu_amd import make_profiles, profiling


def _trace(path, rows):
    keys = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=keys)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(keys, r)))


def test_timed_region_takes_the_last_dispatches(tmp_path):
    rows = []
    # 10 slow "settle" dispatches (2000 ns), then 5 timed ones (1000 ns) every 1500 ns;
    # another kernel interleaved, and rows written out of time order.
    t = 0
    for i in range(10):
        rows.append(("conv", t, t + 2000))
        t += 2500
    for i in range(5):
        rows.append(("conv", t, t + 1000))
        rows.append(("other", t + 1000, t + 1100))
        t += 1500
    rows.reverse()
    p = tmp_path / "run_kernel_trace.csv"
    _trace(p, rows)
    got = profiling.timed_region(str(p), 5)
    assert got["conv"] == {"avg_ns": 1000.0, "spacing_ns": 1500.0, "n": 5}
    assert got["other"]["avg_ns"] == 100.0 and got["other"]["spacing_ns"] == 1500.0
    # a kernel with fewer dispatches than requested is left out
    assert "other" not in profiling.timed_region(str(p), 6)
    assert profiling.timed_region(str(p), 15)["conv"]["avg_ns"] == (10 * 2000 + 5 * 1000) / 15


def test_bench_table(tmp_path, monkeypatch):
    row = {"workload": "w1", "kernel": "igemm_patch cfg=3 f16 N=1", "us": 10.0, "tflops": 1.0,
           "gbs": 2.0, "bound": "hbm", "frac": 0.5, "unfused_us": 20.0,
           "speedup_vs_unfused": 2.0, "split_us": 15.0, "speedup_vs_split": 1.5,
           "act_us": {"relu": 9.0, "gelu": 12.0, "none": 9.0}, "nchw_legs_us": 30.0,
           "nchw_legs_share": 0.66, "train_us": 40.0, "fp8_out_us": 8.0, "fp8_out_gbs": 1.0,
           "residual_us": 12.0, "residual_gbs": 3.0, "packed_us": 9.9,
           "cold_us": {"p10": 11.0, "p50": 12.0, "p90": 13.0, "reps": 100},
           "unfused_cold_us": {"p10": 21.0, "p50": 22.0, "p90": 23.0, "reps": 100},
           "speedup_vs_unfused_cold": 1.83, "predicted_speedup_vs_unfused": 2.2,
           "copy_gbs": 5000.0}
    bare = {"workload": "w0", "kernel": "scalar f32 N=1", "us": 4.0, "tflops": 0.1,
            "gbs": 0.2, "bound": "hbm", "frac": 0.01}
    line = {"steps": 200, "warmup": 20, "settle_ms": 30.0, "value": 2.0, "unit": "GB/s",
            "config": {"workload": "w1", "buffer_sets": 16}, "per_config": [bare, row],
            "roofline": {"frac": 0.5}, "frac_of_copy": 0.9,
            "device": {"name": "gpu", "compute_units": 256},
            "cpu_baseline": {"value": 1.0}}
    js = tmp_path / "b.json"
    js.write_text("log line\n" + json.dumps(line) + "\n")
    monkeypatch.setattr(make_profiles, "PROFILES", str(tmp_path))
    make_profiles.write_bench_table(str(js))
    text = (tmp_path / "bench_per_workload.md").read_text()
    assert "settle 30.0 ms" in text
    lines = text.splitlines()
    w1 = [l for l in lines if l.startswith("w1 |")][0].split(" | ")
    w0 = [l for l in lines if l.startswith("w0 |")][0].split(" | ")
    header = [l for l in lines if l.startswith("workload |")][0].split(" | ")
    assert len(w1) == len(header) == len(w0)
    assert w1[header.index("packed us")] == "9.9"
    assert w1[header.index("cold us p50 (p10-p90)")] == "12.0 (11.0-13.0)"
    assert w1[header.index("x vs unfused cold")] == "1.83"
    assert w0[header.index("cold us p50 (p10-p90)")] == "None"
    assert "against the measured device-copy rate (5000.0 GB/s): 0.9" in text
    assert text.rstrip().endswith("value: 2.0 GB/s (w1)")
