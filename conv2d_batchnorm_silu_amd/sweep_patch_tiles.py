"""Time every tile configuration of the patch-staged implicit GEMM that fits
each stride-1 shape (GPU host only) and compare with the configuration the
plan chooses -> <out>.jsonl and <out>.md.

    python -m conv2d_batchnorm_silu_amd.sweep_patch_tiles --out profiles/patch_tile_sweep

Shapes: k in {1, 3, 5}, C_in in {64, 128}, C_out in {8 .. 256} on 8 x 112 x 112
images (the 7 x 7 ones with C_in = 128 do not fit the patch in LDS there), plus
the 3x3 and 7x7 benchmark layers. Inputs are seeded synthetic tensors; each
configuration is forced through TG_PATCH_CFG (read when a plan is created),
run once, repeated for 10 ms untimed, then timed over `--reps` back-to-back
launches with HIP events.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))


def shapes():
    for k in (1, 3, 5):
        for cin in (64, 128):
            for cout in (8, 16, 24, 32, 48, 64, 128, 256):
                yield dict(name="k%d_c%d_k%d" % (k, cin, cout), N=8, H=112, W=112, C_in=cin,
                           C_out=cout, k=k, pad=k // 2)
    from conv2d_batchnorm_silu_amd.inputs import WORKLOADS
    for name in ("conv3x3_c128_k128", "conv7x7_c64_k64"):
        wl = WORKLOADS[name]
        yield dict(name=name, N=wl.N, H=wl.H, W=wl.W, C_in=wl.C_in, C_out=wl.C_out, k=wl.kh,
                   pad=wl.pad)


def time_plan(torch, plan, x, w, sc, bi, reps):
    y = plan.run(x, w, sc, bi)
    t_end = time.perf_counter() + 0.01
    while time.perf_counter() < t_end:
        plan.run(x, w, sc, bi, out=y)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        plan.run(x, w, sc, bi, out=y)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", default="patch_tile_sweep", help="output path prefix")
    ap.add_argument("--reps", type=int, default=20)
    args = ap.parse_args(argv)

    import torch
    from conv2d_batchnorm_silu_amd import binding as B
    B.library()
    os.environ["TG_CU"] = "0"        # the 1x1 kernels would take some 1x1 shapes
    os.environ["TG_IGEMM_RW"] = "0"
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    rows = []
    with open(args.out + ".jsonl", "w") as jf:
        for s in shapes():
            gen.manual_seed(len(rows) + 1)
            x = torch.randn(s["N"], s["H"], s["W"], s["C_in"], device=dev, generator=gen).half()
            w = (torch.randn(s["C_out"], s["k"], s["k"], s["C_in"], device=dev, generator=gen) /
                 (s["k"] * s["k"] * s["C_in"]) ** 0.5).half()
            sc = torch.ones(s["C_out"], device=dev)
            bi = torch.zeros(s["C_out"], device=dev)
            mk = lambda: B.ConvBnSilu(s["N"], s["H"], s["W"], s["C_in"], s["C_out"], s["k"],
                                      s["k"], 1, s["pad"], "f16", "igemm")
            os.environ.pop("TG_PATCH_CFG", None)
            chosen = mk().describe()
            if not chosen.startswith("igemm_patch"):
                continue
            us = {}
            for cfg in range(10):
                os.environ["TG_PATCH_CFG"] = str(cfg)
                plan = mk()
                if not plan.describe().startswith("igemm_patch cfg=%d " % cfg):
                    continue  # this tile does not fit the shape
                us[cfg] = round(time_plan(torch, plan, x, w, sc, bi, args.reps), 2)
            os.environ.pop("TG_PATCH_CFG", None)
            row = dict(s, chosen=int(chosen.split("cfg=")[1].split()[0]), us=us)
            rows.append(row)
            jf.write(json.dumps(row) + "\n")
            jf.flush()
            print(json.dumps(row), flush=True)
    lines = ["# Patch-staged implicit GEMM: every tile configuration per stride-1 shape "
             "(one MI355X)",
             "# command: python -m conv2d_batchnorm_silu_amd.sweep_patch_tiles --out "
             "profiles/patch_tile_sweep",
             "# us per launch (HIP events, %d back-to-back launches after 10 ms untimed); "
             "'-' = the tile does not fit the shape" % args.reps,
             "",
             "shape | N H W | " + " | ".join("cfg %d" % c for c in range(10)) +
             " | chosen | chosen / fastest",
             "---|---|" + "---|" * 10 + "---|---"]
    ratios = []
    for r in rows:
        best = min(r["us"].values())
        ratio = r["us"][r["chosen"]] / best
        ratios.append(ratio)
        lines.append("%s | %d %d %d | %s | %d | %.3f" % (
            r["name"], r["N"], r["H"], r["W"],
            " | ".join(str(r["us"].get(c, "-")) for c in range(10)), r["chosen"], ratio))
    if ratios:
        lines += ["", "chosen = fastest on %d of %d shapes; worst chosen / fastest %.3f" % (
            sum(1 for q in ratios if q == 1.0), len(ratios), max(ratios))]
    with open(args.out + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote %s.md" % args.out, file=sys.stderr)


if __name__ == "__main__":
    main()
