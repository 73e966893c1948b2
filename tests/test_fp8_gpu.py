"""GPU parity of the fp8 (OCP E4M3) output cast in the epilogue
(tg_conv_bn_act_create_out) in every kernel family, against the oracle's
fp64 result. Bar per element: |gpu - oracle| <= (0.5 + 2^-7) E4M3 spacings
at the oracle's value, spacing 2^(max(floor(log2|o|), -6) - 3):
round-to-nearest gives at most half a spacing; the kernels round the fp32
epilogue result to fp16 first (their output tiles are fp16), which adds at
most 2^-8 of a spacing (derivation at FP8_BAR). Most elements must equal the
oracle's own E4M3 rounding exactly (at least 99%). A decode of the bytes as
fp8 in another layout (FNUZ) would fail both bars by a factor of 2.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from conv2d_batchnorm_silu_amd import binding as B
from conv2d_batchnorm_silu_amd.inputs import WORKLOADS, Workload, make_inputs

from gpu_cases import note

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def run_fp8(wl, act="silu", kernel="auto"):
    d = make_inputs(wl)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items() if k != "eps"}
    scale, bias = B.bn_fold(t["gamma"], t["beta"], t["mean"], t["var"], float(d["eps"]))
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype, kernel, act=act, out_dtype="f8")
    note("%s fp8 act=%s kernel=%s plan=%s" % (wl.name, act, kernel, plan.describe()))
    y = plan.run(t["x"], t["w"], scale, bias)
    torch.cuda.synchronize()
    assert y.dtype == torch.float8_e4m3fn
    return d, plan, y.float().cpu().numpy().astype(np.float64)


# Half an E4M3 spacing for the final rounding, plus the fp16 rounding before
# it (fp16 keeps 7 more mantissa bits than E4M3: at most 2^-8 of a spacing,
# also when that rounding lands on an E4M3 midpoint and the tie goes to even)
# and the fp32 arithmetic (about 1e-6 relative, under 2^-16 of a spacing):
# 0.5 + 2^-8 + 2^-16 < 0.5 + 2^-7.
FP8_BAR = 0.5 + 2.0 ** -7


def check_fp8(wl, got, ref, what):
    assert not np.isnan(got).any(), what
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    spacing = np.exp2(np.maximum(e, -6.0) - 3.0)
    err = np.abs(got - ref)
    worst = float((err / spacing).max())
    exact = float((got == oracle.round_fp8_e4m3(ref)).mean())
    note("%s: max error %.3g spacings, %.4f equal to the oracle's rounding" % (what, worst, exact))
    assert worst <= FP8_BAR, what
    assert exact >= 0.99, what


SHAPES = [
    WORKLOADS["conv1x1_c64_k256"].scaled(N=1, H=13, W=17),
    WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=17, W=15),
    WORKLOADS["conv7x7_c64_k64"].scaled(N=1, H=13, W=11),
    WORKLOADS["stem3x3s2_k24"].scaled(N=2, H=40, W=36),
    Workload("fp8_rw_c16", 90, 2, 11, 9, 16, 48, 1, 1, 1, 0, "f16"),
    Workload("fp8_cout7", 91, 2, 9, 9, 16, 7, 3, 3, 2, 1, "f16"),
]


@pytest.mark.parametrize("act", ["silu", "relu"])
@pytest.mark.parametrize("kernel", ["auto", "scalar", "igemm", "tiled"])
def test_fp8_shapes(kernel, act):
    ran = 0
    for wl in SHAPES:
        try:
            B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                         wl.dtype, kernel, act=act, out_dtype="f8")
        except B.TgError:
            continue
        d, plan, got = run_fp8(wl, act, kernel)
        ref = oracle.conv_bn_act(d["x"], d["w"], d["gamma"], d["beta"], d["mean"], d["var"],
                                 float(d["eps"]), wl.stride, wl.pad, act)
        check_fp8(wl, got, ref, "%s/%s/%s" % (wl.name, act, kernel))
        ran += 1
    assert ran >= 2


VARIANTS = [
    ({"cu": "0"}, WORKLOADS["conv1x1_c64_k256"].scaled(N=1, H=13, W=17), "igemm_rw"),
    ({"cu": "0", "igemm_rw": "0", "igemm_patch": "0"},
     WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=17, W=15), "igemm_dma"),
    ({"cu": "0", "igemm_rw": "0", "igemm_patch": "0", "igemm_dma": "0"},
     WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=17, W=15), "igemm"),
    ({"stem": "0"}, WORKLOADS["stem3x3s2_k16"].scaled(N=2, H=40, W=40), "tiled_mfma_pipe"),
    ({"stem": "0", "tm_pipe": "0"}, WORKLOADS["stem3x3s2_k16"].scaled(N=2, H=40, W=40),
     "tiled_mfma"),
    ({"stem": "0", "tiled_mfma": "0"},
     WORKLOADS["stem3x3s2_k16"].scaled(N=2, H=40, W=36), "tiled"),
]


@pytest.mark.parametrize("env,wl,prefix", VARIANTS, ids=[v[2] for v in VARIANTS])
def test_fp8_variants(tune, env, wl, prefix):
    tune(**env)
    d, plan, got = run_fp8(wl)
    assert plan.describe().startswith(prefix), plan.describe()
    ref = oracle.conv_bn_silu(d["x"], d["w"], d["gamma"], d["beta"], d["mean"], d["var"],
                              float(d["eps"]), wl.stride, wl.pad)
    check_fp8(wl, got, ref, "%s/%s" % (wl.name, prefix))


@pytest.mark.parametrize("name", ["conv1x1_c64_k256", "conv3x3_c128_k128", "stem3x3s2_k16",
                                  "stem3x3s2_k24", "conv7x7_c64_k64"])
def test_fp8_full_size(name):
    """Every output of the full workload in the dispatched configuration."""
    wl = WORKLOADS[name]
    d, plan, got = run_fp8(wl)
    ref = oracle.conv_bn_silu(d["x"], d["w"], d["gamma"], d["beta"], d["mean"], d["var"],
                              float(d["eps"]), wl.stride, wl.pad)
    check_fp8(wl, got, ref, "%s full" % name)


def test_fp8_rejected_where_unsupported():
    wl = WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=8, W=8)
    for kernel in ("unfused", "split"):
        with pytest.raises(B.TgError):
            B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                         wl.dtype, kernel, out_dtype="f8")
    t0 = WORKLOADS["tiny_f32_3x3"]
    with pytest.raises(B.TgError):
        B.ConvBnSilu(t0.N, t0.H, t0.W, t0.C_in, t0.C_out, t0.kh, t0.kw, t0.stride, t0.pad, "f32",
                     out_dtype="f8")
