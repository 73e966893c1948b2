"""GPU parity of the residual add in the epilogue
(tg_conv_bn_silu_run_residual): y = act(BN(conv)) + r in every kernel
family, against the oracle's conv_bn_act_residual. Bars: the north-star
tolerance (fp16 |gpu - oracle| <= 1e-2 * max(1, |oracle|), fp32 1e-4) and,
derived from the arithmetic, two roundings for fp16 -- the activated value
to fp16, then the fp32 sum to fp16 -- so |gpu - oracle| <= 2^-10 * max(1,
|act|, |oracle|) plus the fp32 epilogue's ~1e-6; fp32: 1e-5 * max(1, |act|,
|oracle|)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from conv2d_batchnorm_silu_amd import binding as B
from conv2d_batchnorm_silu_amd.inputs import WORKLOADS, Workload, make_inputs

from gpu_cases import note

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def run_res(wl, act="silu", kernel="auto", seed=0):
    d = make_inputs(wl)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items() if k != "eps"}
    scale, bias = B.bn_fold(t["gamma"], t["beta"], t["mean"], t["var"], float(d["eps"]))
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype, kernel, act=act)
    npdt = np.float16 if wl.dtype == "f16" else np.float32
    r = np.random.default_rng(1000 + seed).normal(size=plan.y_shape).astype(npdt)
    rt = torch.from_numpy(r).cuda()
    note("%s residual act=%s kernel=%s plan=%s" % (wl.name, act, kernel, plan.describe()))
    y = plan.run(t["x"], t["w"], scale, bias, residual=rt)
    torch.cuda.synchronize()
    return d, r, plan, y.float().cpu().numpy().astype(np.float64)


def check_res(wl, d, r, got, act, what):
    args = (d["gamma"], d["beta"], d["mean"], d["var"], float(d["eps"]), wl.stride, wl.pad, act)
    a = oracle.conv_bn_act(d["x"], d["w"], *args)
    o = a + r.astype(np.float64)
    assert not np.isnan(got).any(), what
    tol = 1e-2 if wl.dtype == "f16" else 1e-4
    tight = 2.0 ** -10 + 1e-6 if wl.dtype == "f16" else 1e-5
    err = np.abs(got - o)
    worst = float((err / np.maximum(1.0, np.abs(o))).max())
    worst_t = float((err / np.maximum.reduce([np.ones_like(o), np.abs(a), np.abs(o)])).max())
    note("%s: max scaled error %.3g (derived bound %.3g)" % (what, worst, worst_t))
    assert worst <= tol, what
    assert worst_t <= tight, what


SHAPES = [
    WORKLOADS["tiny_f32_3x3"],
    WORKLOADS["conv1x1_c64_k256"].scaled(N=1, H=13, W=17),
    WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=17, W=15),
    WORKLOADS["conv7x7_c64_k64"].scaled(N=1, H=13, W=11),
    WORKLOADS["stem3x3s2_k24"].scaled(N=2, H=40, W=36),
    Workload("res_rw_c16", 95, 2, 11, 9, 16, 48, 1, 1, 1, 0, "f16"),
    Workload("res_cout7", 96, 2, 9, 9, 16, 7, 3, 3, 2, 1, "f16"),
]


@pytest.mark.parametrize("act", ["silu", "relu"])
@pytest.mark.parametrize("kernel", ["auto", "scalar", "igemm", "tiled"])
def test_residual_shapes(kernel, act):
    ran = 0
    for i, wl in enumerate(SHAPES):
        try:
            B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                         wl.dtype, kernel, act=act)
        except B.TgError:
            continue
        d, r, plan, got = run_res(wl, act, kernel, seed=i)
        check_res(wl, d, r, got, act, "%s/%s/%s" % (wl.name, act, kernel))
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
def test_residual_variants(tune, env, wl, prefix):
    tune(**env)
    d, r, plan, got = run_res(wl)
    assert plan.describe().startswith(prefix), plan.describe()
    check_res(wl, d, r, got, "silu", "%s/%s" % (wl.name, prefix))


def test_residual_full_size_headline():
    """The 1x1 layer at full size in the dispatched configuration (the one
    workgroup per CU kernel's residual instantiation), every output."""
    wl = WORKLOADS["conv1x1_c64_k256"]
    d, r, plan, got = run_res(wl)
    assert plan.describe().startswith("igemm_cu")
    check_res(wl, d, r, got, "silu", "%s full" % wl.name)


def test_residual_rejected_where_unsupported():
    wl = WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=8, W=8)
    d = make_inputs(wl)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items() if k != "eps"}
    scale, bias = B.bn_fold(t["gamma"], t["beta"], t["mean"], t["var"], float(d["eps"]))
    for kw in ({"kernel": "split"}, {"kernel": "unfused"}, {"out_dtype": "f8"}):
        plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride,
                            wl.pad, wl.dtype, **kw)
        r = torch.zeros(plan.y_shape, dtype=torch.float16, device="cuda")
        with pytest.raises((B.TgError, ValueError)):
            plan.run(t["x"], t["w"], scale, bias, residual=r)
