"""Measured MI355X peaks: HBM streaming, fp16 MFMA, VALU/transcendental and LDS read rates.

    python -m conv2d_batchnorm_silu_amd.peaks [--out profiles/peaks_mi355x]

Builds libtgpeaks.so from peaks.hip (hipcc, gfx950) next to this file, runs
each microbenchmark after a clock-settling phase and times it with HIP events
on the launch stream; prints one JSON object and, with --out, writes
<out>.md and <out>.json. The fused kernels' roofline fractions use the
published peaks (HBM 8 TB/s, dense fp16 MFMA 2516.6 TFLOP/s); these numbers
say how much of each a kernel of this library can reach.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "peaks.hip")
LIB = os.path.join(PKG, "libtgpeaks.so")
CUS = 256
CLOCK_GHZ = 2.4  # MI355X peak engine clock, for per-clock figures


def build() -> str:
    sys.path.insert(0, ROOT)
    from conv2d_batchnorm_silu_amd.build import ARCH, hipcc
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", tmp, SRC]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _lib():
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(LIB)
    vp, i, ll = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    lib.tgp_copy.argtypes = [vp, vp, ll, i, vp]
    lib.tgp_copy_dma.argtypes = [vp, vp, ll, i, vp]
    lib.tgp_read.argtypes = [vp, ll, vp, i, vp]
    lib.tgp_write.argtypes = [vp, ll, i, i, vp]
    lib.tgp_mfma.argtypes = [i, i, i, i, vp, vp]
    lib.tgp_lds.argtypes = [i, i, i, vp, vp]
    lib.tgp_lds_stride.argtypes = [i, i, i, i, vp, vp]
    lib.tgp_valu.argtypes = [i, i, i, i, vp, vp]
    lib.tgp_mfma_lds.argtypes = [i, i, i, vp, vp, vp]
    lib.tgp_lds_pattern.argtypes = [i, i, i, i, vp, vp]
    lib.tgp_vmem_batch.argtypes = [i, i, vp, ctypes.c_ulonglong, i, i, i, vp, vp]
    return lib


def _time(torch, fn, reps, settle_ms=30.0):
    """ms per call of fn() (returns a hipError_t) after settle_ms of calls."""
    t_end = time.perf_counter() + settle_ms / 1e3
    while time.perf_counter() < t_end:
        for _ in range(10):
            assert fn() == 0
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        assert fn() == 0
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure() -> dict:
    import torch
    lib = _lib()
    s = torch.cuda.current_stream().cuda_stream
    out = torch.zeros(16, dtype=torch.float32, device="cuda")
    res = {"device": torch.cuda.get_device_name(0), "hip": torch.version.hip,
           "compute_units": torch.cuda.get_device_properties(0).multi_processor_count}
    nbytes = 1 << 30
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    grid = CUS * 8
    ms = _time(torch, lambda: lib.tgp_copy(a.data_ptr(), b.data_ptr(), nbytes, grid, s), 10)
    res["hbm_copy_gbs"] = round(2 * nbytes / ms / 1e6, 1)
    ms = _time(torch, lambda: lib.tgp_copy_dma(a.data_ptr(), b.data_ptr(), nbytes, grid, s), 10)
    res["hbm_copy_dma_gbs"] = round(2 * nbytes / ms / 1e6, 1)
    ms = _time(torch, lambda: lib.tgp_read(a.data_ptr(), nbytes, out.data_ptr(), grid, s), 10)
    res["hbm_read_gbs"] = round(nbytes / ms / 1e6, 1)
    for nt in (0, 1):
        ms = _time(torch, lambda: lib.tgp_write(b.data_ptr(), nbytes, nt, grid, s), 10)
        res["hbm_write_%s_gbs" % ("nt" if nt else "plain")] = round(nbytes / ms / 1e6, 1)
    # The same copy at the HBM-bound layers' sizes (bytes read + written =
    # the layer's algorithmic bytes): the rate a streaming kernel of that
    # size can reach,
    # launch and ramp included (grid: 8 workgroups of 256 per CU, capped by
    # the 16-byte elements).
    # Successive calls take successive slices of the 1 GB buffers, as the
    # bench rotates its input and output copies, so that each call reads
    # and writes HBM rather than the last-level cache.
    for name, moved in (("conv1x1_c64_k256", 64_260_096), ("stem3x3s2_k16", 44_958_688),
                        ("stem3x3s2_k24", 57_804_240)):
        half = moved // 2 // 256 * 256
        g = min(CUS * 8, (half // 16 + 255) // 256)
        nslices = nbytes // half
        ctr = [0]

        def rotating_copy():
            k = ctr[0] % nslices
            ctr[0] += 1
            return lib.tgp_copy(a.data_ptr() + k * half, b.data_ptr() + k * half, half, g, s)

        ms = _time(torch, rotating_copy, 4 * nslices)
        res["copy_%s_us" % name] = round(ms * 1e3, 2)
        res["copy_%s_gbs" % name] = round(2 * half / ms / 1e6, 1)
    del a, b
    iters = 4000
    for shape, name, flop_per_wave_iter in ((0, "16x16x32", 8 * 16384), (1, "32x32x16", 4 * 32768)):
        for waves_per_simd in (1, 2):
            block = 256 * waves_per_simd
            g = CUS
            ms = _time(torch, lambda: lib.tgp_mfma(shape, iters, g, block, out.data_ptr(), s), 5)
            flop = g * (block // 64) * iters * flop_per_wave_iter
            res["mfma_f16_%s_%dw_tflops" % (name, waves_per_simd)] = round(flop / ms / 1e9, 1)
    # The implicit-GEMM step (4 x 7 MFMAs per wave, 4 waves per CU): clocks
    # per step with the MFMAs alone, with the 7 pixel-fragment LDS reads,
    # and with the 4 filter-fragment loads as well.
    g = torch.zeros(4096, dtype=torch.float16, device="cuda")
    for mode, name in ((0, "mfma"), (1, "mfma_lds"), (2, "mfma_lds_load")):
        iters = 2000
        ms = _time(torch, lambda: lib.tgp_mfma_lds(mode, iters, CUS, g.data_ptr(), out.data_ptr(), s), 5)
        res["step_%s_clk" % name] = round(ms * 1e-3 * CLOCK_GHZ * 1e9 / (iters * 2), 1)
    # VALU: fma, exp and rcp, lane-operations per clock per CU (8 per lane
    # and iteration, extra multiply/add of the exp/rcp chains not counted).
    valu_iters = 20000
    for op, name in ((0, "fma"), (1, "exp"), (2, "rcp")):
        for waves_per_simd in (1, 2):
            block = 256 * waves_per_simd
            ms = _time(torch, lambda: lib.tgp_valu(op, valu_iters, CUS, block, out.data_ptr(), s), 5)
            ops = CUS * block * valu_iters * 8
            res["valu_%s_%dw_ops_per_clk_cu" % (name, waves_per_simd)] = round(
                ops / (ms / 1e3) / (CUS * CLOCK_GHZ * 1e9), 1)
    lds_iters = 20000
    for waves in (4, 8):
        block = 64 * waves
        ms = _time(torch, lambda: lib.tgp_lds(lds_iters, CUS, block, out.data_ptr(), s), 5)
        nb = CUS * waves * lds_iters * 8 * 1024
        tbs = nb / ms / 1e9
        res["lds_read_b128_%dw_tbs" % waves] = round(tbs, 2)
        res["lds_read_b128_%dw_bytes_per_clk_cu" % waves] = round(
            tbs * 1e12 / (CUS * CLOCK_GHZ * 1e9), 1)
    # Fragment-read pattern: 16 rows of `stride` bytes, 4 pieces each.
    for stride in (128, 144, 160, 176, 192, 256, 272, 288):
        ms = _time(torch, lambda: lib.tgp_lds_stride(lds_iters, stride, CUS, 256,
                                                     out.data_ptr(), s), 5)
        nb = CUS * 4 * lds_iters * 8 * 1024
        res["lds_frag_stride%d_bytes_per_clk_cu" % stride] = round(
            nb / ms / 1e9 * 1e12 / (CUS * CLOCK_GHZ * 1e9), 1)
    # One wave's batch of n 1 KB loads, then a wait: ns per batch, from an
    # L2-resident 1 MB window and from a 1 GB window (HBM), one wave per CU
    # and eight.
    big = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(3)
    vb_iters = 400
    for window, wname in ((1 << 20, "l2"), (1 << 30, "hbm")):
        for waves in (1, 8):
            for mode, mname in ((0, "lds"), (1, "vgpr")):
                for n in (1, 4, 16):
                    ms = _time(torch, lambda: lib.tgp_vmem_batch(mode, n, big.data_ptr(), window, vb_iters,
                                                                  CUS, waves, out.data_ptr(), s), 3)
                    res["vmem_batch_%s_%s_%dw_n%d_ns" % (mname, wname, waves, n)] = round(
                        ms * 1e6 / vb_iters, 1)
    del big
    # Fragment layouts (peaks.hip, pk_lds_pattern): 8 waves per CU, 12 reads
    # in flight per wave; bytes per clock per CU.
    pat_iters = 4000
    patterns = [("linear", 0, 0)]
    for stride in (144, 160, 176, 272, 288):
        patterns.append(("patch_stride%d" % stride, 1, stride))
        patterns.append(("patch_stride%d_wrap" % stride, 2, stride))
    patterns += [("ring64_swz_r1", 3, 0), ("ring64_swz_r2", 4, 0), ("ring64_swz_r1r2", 5, 0),
                 ("ring128_swz_r1_lo", 6, 0), ("ring128_swz_r1_hi", 6, 1),
                 ("ring128_swz_r7r3_lo", 7, 0), ("ring128_swz_r7r3_hi", 7, 1)]
    for name, mode, prm in patterns:
        ms = _time(torch, lambda: lib.tgp_lds_pattern(pat_iters, mode, prm, CUS, out.data_ptr(), s), 5)
        nb = CUS * 8 * pat_iters * 12 * 1024
        res["lds_pattern_%s_bytes_per_clk_cu" % name] = round(
            nb / ms / 1e9 * 1e12 / (CUS * CLOCK_GHZ * 1e9), 1)
    return res


def write(res: dict, out: str):
    cmd = "python -m conv2d_batchnorm_silu_amd.peaks --out %s" % os.path.relpath(out, ROOT)
    lines = ["# Measured MI355X peaks (microbenchmarks in conv2d_batchnorm_silu_amd/peaks.hip)",
             "# command: " + cmd,
             "# HIP events over back-to-back launches after 30 ms of settling calls;",
             "# published: HBM 8000 GB/s, dense fp16 MFMA 2516.6 TFLOP/s",
             "",
             "| rate | value |", "|---|---|"]
    for k, v in res.items():
        lines.append("| %s | %s |" % (k, v))
    with open(out + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(out + ".json", "w") as f:
        json.dump(res, f, indent=1)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", default=None, help="write <out>.md and <out>.json")
    ap.add_argument("--build-only", action="store_true")
    args = ap.parse_args()
    if args.build_only:
        print(build())
        return
    res = measure()
    print(json.dumps(res))
    if args.out:
        write(res, os.path.join(ROOT, args.out) if not os.path.isabs(args.out) else args.out)


if __name__ == "__main__":
    main()
