"""Re-measure the shape -> kernel dispatch table on the GPU this runs on.

Times every kernel that serves a shape (scalar, tiled, igemm, each forced)
and the default dispatch over a grid of layer shapes, and writes one JSON
line per shape plus a markdown summary: the fastest kernel, what the
default table picks, and how far it is from the fastest. This is the
measurement behind the default (MI355X) table in csrc/api.hip; the page's
own thresholds ("Fusing an Epilogue", teenygrad docs, "Three kernels for one
operation") were set on other hardware.

Grid: k in {1, 3, 5, 7} (pad k//2), stride in {1, 2}, C_in in {3, 16, 64,
128}, C_out in {8, 12, 16, 20, 24, 32, 48, 64, 128, 256}; N = 8 and H = W =
112 (stride 1) or 224 (stride 2), i.e. 100,352 output pixels per channel.
Inputs are device-side random fp16 tensors (correctness is the tests' job).

    python -m conv2d_batchnorm_silu_amd.sweep_dispatch --out profiles/dispatch_sweep

With --patch-tiles it times every tile configuration of the patch-staged
implicit GEMM on the stride-1 shapes it serves instead (the data behind the
tile cost model in csrc/igemm_patch.hip):

    python -m conv2d_batchnorm_silu_amd.sweep_dispatch --patch-tiles --reps 20 \
        --out profiles/patch_tile_sweep
"""
import argparse
import json
import math
import os
import sys
import time

KERNELS = ("scalar", "tiled", "igemm")
SCALAR_MAX_GFLOP = 40.0  # the scalar kernel is not timed beyond this (seconds per shape)


def shapes():
    for k in (1, 3, 5, 7):
        for s in (1, 2):
            for cin in (3, 16, 64, 128):
                for cout in (8, 12, 16, 20, 24, 32, 48, 64, 128, 256):
                    hw = 112 if s == 1 else 224
                    yield dict(N=8, H=hw, W=hw, C_in=cin, C_out=cout, k=k, stride=s, pad=k // 2)


def time_plan(torch, plan, x, w, sc, bi, y, reps):
    # 5 ms of untimed calls first: the clocks drop while the host builds the
    # next shape's inputs (the benchmark settles them the same way).
    t_end = time.perf_counter() + 0.005
    plan.run(x, w, sc, bi, out=y)
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
    return e0.elapsed_time(e1) * 1e3 / reps  # us


def tile_shapes():
    """Stride-1 shapes for the patch-staged kernel's tile sweep: k in {1, 3,
    5}, C_in in {64, 128}, C_out in {8 .. 256} on 8 x 112 x 112 images, plus
    the 3x3 and 7x7 benchmark layers."""
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


def patch_tiles(out, reps):
    """Every tile configuration of the patch-staged implicit GEMM that fits
    each shape of tile_shapes(), forced with the tuning key patch_cfg (the 1x1
    kernels switched off with cu=0, igemm_rw=0), against the configuration
    the plan chooses -> <out>.jsonl and <out>.md."""
    import torch
    from conv2d_batchnorm_silu_amd import binding as B
    B.library()
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    base = {"cu": 0, "igemm_rw": 0}
    rows = []
    with open(out + ".jsonl", "w") as jf:
        for s in tile_shapes():
            gen.manual_seed(len(rows) + 1)
            x = torch.randn(s["N"], s["H"], s["W"], s["C_in"], device=dev, generator=gen).half()
            w = (torch.randn(s["C_out"], s["k"], s["k"], s["C_in"], device=dev, generator=gen) /
                 (s["k"] * s["k"] * s["C_in"]) ** 0.5).half()
            sc = torch.ones(s["C_out"], device=dev)
            bi = torch.zeros(s["C_out"], device=dev)
            y = torch.empty(s["N"], s["H"] + 2 * s["pad"] - s["k"] + 1,
                            s["W"] + 2 * s["pad"] - s["k"] + 1, s["C_out"], device=dev).half()

            def mk(extra):
                return B.ConvBnSilu(s["N"], s["H"], s["W"], s["C_in"], s["C_out"], s["k"], s["k"],
                                    1, s["pad"], "f16", "igemm", tuning=dict(base, **extra))
            chosen = mk({}).describe()
            if not chosen.startswith("igemm_patch"):
                continue
            us = {}
            for cfg in range(10):
                plan = mk({"patch_cfg": cfg})
                if not plan.describe().startswith("igemm_patch cfg=%d " % cfg):
                    continue  # this tile does not fit the shape
                us[cfg] = round(time_plan(torch, plan, x, w, sc, bi, y, reps), 2)
            row = dict(s, chosen=int(chosen.split("cfg=")[1].split()[0]), us=us)
            rows.append(row)
            jf.write(json.dumps(row) + "\n")
            jf.flush()
            print(json.dumps(row), flush=True)
    lines = ["# Patch-staged implicit GEMM: every tile configuration per stride-1 shape "
             "(one MI355X)",
             "# command: python -m conv2d_batchnorm_silu_amd.sweep_dispatch --patch-tiles --out "
             "%s --reps %d" % (out, reps),
             "# us per launch (HIP events over %d back-to-back launches after 5 ms untimed); "
             "'-' = the tile does not fit the shape" % reps,
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
        lines += ["", "chosen = fastest on %d of %d shapes; within 10%% on %d; worst chosen / "
                  "fastest %.3f" % (sum(1 for q in ratios if q == 1.0), len(ratios),
                                    sum(1 for q in ratios if q <= 1.10), max(ratios))]
    with open(out + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote %s.md" % out, file=sys.stderr)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", default="dispatch_sweep", help="output path prefix (.jsonl, .md)")
    ap.add_argument("--patch-tiles", action="store_true",
                    help="time every tile of the patch-staged kernel instead (patch_tiles())")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--limit", type=int, default=0, help="only the first N shapes (0: all)")
    ap.add_argument("--from-jsonl", default=None,
                    help="re-render <out>.md from this JSON-lines file of an earlier sweep")
    ap.add_argument("--gpu", default=None, help="device name for the header (--from-jsonl)")
    args = ap.parse_args(argv)
    if args.patch_tiles:
        patch_tiles(args.out, args.reps)
        return 0
    if args.from_jsonl:
        with open(args.from_jsonl) as f:
            rows = [json.loads(l) for l in f if l.strip()]
        write_summary(rows, args.out + ".md", args.gpu, rendered_from=True)
        return 0

    import torch
    from conv2d_batchnorm_silu_amd import binding as B

    dev = torch.device("cuda")
    rows = []
    t_start = time.time()
    for i, sh in enumerate(shapes()):
        if args.limit and i >= args.limit:
            break
        N, H, W, cin, cout, k, s, p = (sh[a] for a in ("N", "H", "W", "C_in", "C_out", "k",
                                                     "stride", "pad"))
        P = (H + 2 * p - k) // s + 1
        Q = (W + 2 * p - k) // s + 1
        gflop = 2.0 * N * P * Q * cout * k * k * cin / 1e9
        x = torch.randn(N, H, W, cin, device=dev, dtype=torch.float16)
        w = (torch.randn(cout, k, k, cin, device=dev) / math.sqrt(k * k * cin)).half()
        sc = torch.ones(cout, device=dev)
        bi = torch.zeros(cout, device=dev)
        y = torch.empty(N, P, Q, cout, device=dev, dtype=torch.float16)
        row = dict(sh, gflop=round(gflop, 3), us={})
        for kern in KERNELS + ("auto",):
            if kern == "scalar" and gflop > SCALAR_MAX_GFLOP:
                row["us"][kern] = None
                continue
            try:
                plan = B.ConvBnSilu(N, H, W, cin, cout, k, k, s, p, "f16", kern)
            except Exception:
                row["us"][kern] = None  # the kernel does not serve this shape
                continue
            reps = args.reps if kern != "scalar" or gflop < 4 else 2
            try:
                row["us"][kern] = round(time_plan(torch, plan, x, w, sc, bi, y, reps), 2)
            except Exception as e:  # a launch-time refusal (e.g. alignment): not served
                print("[sweep] %s refused: %s" % (kern, e), flush=True)
                row["us"][kern] = None
                continue
            if kern == "auto":
                row["auto"] = B.kernel_name(plan.kernel)
                row["auto_describe"] = plan.describe()
        timed = {kk: v for kk, v in row["us"].items() if kk != "auto" and v is not None}
        row["best"] = min(timed, key=timed.get)
        row["auto_over_best"] = round(row["us"]["auto"] / timed[row["best"]], 3)
        rows.append(row)
        print("[sweep] %3d k=%d s=%d C_in=%3d C_out=%3d  %s  best=%s auto=%s (%.2fx)  %.0fs" % (
            i, k, s, cin, cout, " ".join("%s=%s" % (kk, v) for kk, v in row["us"].items()),
            row["best"], row["auto"], row["auto_over_best"], time.time() - t_start), flush=True)
        del x, w, y
        torch.cuda.empty_cache()

    with open(args.out + ".jsonl", "w") as f:
        for r in rows:
            f.write(json.dumps(r) + "\n")
    write_summary(rows, args.out + ".md")


def choice_ratio(r):
    """Forced time of the kernel the default picks over the fastest forced
    time: how good the choice is, free of the run-to-run noise between the
    default's own timing and the forced timing of the same kernel."""
    kind = r["auto"].replace("conv2d_bn_silu_", "")
    u = r["us"]
    if u.get(kind) is None or u.get(r["best"]) is None:
        return r["auto_over_best"]
    return round(u[kind] / u[r["best"]], 3)


def write_summary(rows, path, gpu=None, rendered_from=False):
    if gpu is None:
        import torch
        gpu = torch.cuda.get_device_name(0) if torch.cuda.is_available() else "?"
    L = ["# Dispatch sweep: every kernel that serves a shape, timed on %s" % gpu,
         "# command: python -m conv2d_batchnorm_silu_amd.sweep_dispatch --out profiles/dispatch_sweep",
         "# times: us per launch (HIP events, back to back, same input); '-' = kernel does not serve "
         "the shape or the scalar kernel was not timed (> %.0f GFLOP)" % SCALAR_MAX_GFLOP,
         "",
         "# (this summary re-rendered from that run's JSON lines with --from-jsonl)"
         if rendered_from else "#",
         "# choice / fastest: the forced time of the kernel the default picks over the fastest "
         "forced time; default / fastest: the default plan's own timing over the same (its "
         "excess over the choice ratio is run-to-run noise of the short timings)",
         "",
         "k | s | C_in | C_out | GFLOP | scalar | tiled | igemm | default picks | choice / fastest "
         "| default / fastest"]
    L.append("|".join(["---"] * 11))
    for r in rows:
        u = r["us"]
        f = lambda v: "-" if v is None else "%.1f" % v
        L.append("%d | %d | %d | %d | %.2f | %s | %s | %s | %s | %.2f | %.2f" % (
            r["k"], r["stride"], r["C_in"], r["C_out"], r["gflop"], f(u.get("scalar")),
            f(u.get("tiled")), f(u.get("igemm")), r["auto"], choice_ratio(r),
            r["auto_over_best"]))
    within = sum(1 for r in rows if choice_ratio(r) <= 1.10)
    best = sum(1 for r in rows if choice_ratio(r) <= 1.0)
    raw = sum(1 for r in rows if r["auto_over_best"] <= 1.10)
    worst = sorted(rows, key=lambda r: -choice_ratio(r))[:10]
    L += ["", "default picks the fastest kernel on %d of %d shapes and one within 10%% of it on %d; "
          "the default plan's own timing is within 10%% of the fastest on %d; worst choices:" % (
              best, len(rows), within, raw)]
    for r in worst:
        L.append("  k=%d s=%d C_in=%d C_out=%d: default %s %.2fx the fastest (%s)" % (
            r["k"], r["stride"], r["C_in"], r["C_out"], r["auto"], choice_ratio(r), r["best"]))
    with open(path, "w") as f:
        f.write("\n".join(L) + "\n")


if __name__ == "__main__":
    sys.exit(main())
