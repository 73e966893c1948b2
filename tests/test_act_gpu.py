"""GPU parity of the epilogue activations other than SiLU (ReLU, exact GELU,
BatchNorm only) through tg_conv_bn_act_create + run, against the oracle's
conv_bn_act, in every kernel family (each forced through its switch). Bars as
for SiLU: fp16 |gpu - oracle| <= 1e-2 * max(1, |oracle|), fp32 1e-4, and the
tighter arithmetic bound of gpu_cases (fp16 output rounding, 2e-3; fp32,
1e-5); no NaN."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from conv2d_batchnorm_silu_amd import binding as B
from conv2d_batchnorm_silu_amd.inputs import WORKLOADS, Workload, make_inputs

from gpu_cases import compare, note

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ACTS = ["relu", "gelu", "none"]


def run_act(wl, act, kernel="auto"):
    d = make_inputs(wl)
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in d.items() if k != "eps"}
    scale, bias = B.bn_fold(t["gamma"], t["beta"], t["mean"], t["var"], float(d["eps"]))
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype, kernel, act=act)
    note("%s act=%s kernel=%s plan=%s" % (wl.name, act, kernel, plan.describe()))
    y = plan.run(t["x"], t["w"], scale, bias)
    torch.cuda.synchronize()
    return d, plan, y


def check_act(wl, act, kernel="auto"):
    d, plan, y = run_act(wl, act, kernel)
    ref = oracle.conv_bn_act(d["x"], d["w"], d["gamma"], d["beta"], d["mean"], d["var"],
                             float(d["eps"]), wl.stride, wl.pad, act)
    compare(y.cpu().numpy(), ref, wl.dtype, "%s/%s/%s" % (wl.name, act, kernel))
    return plan


SHAPES = [
    WORKLOADS["tiny_f32_3x3"],
    WORKLOADS["conv1x1_c64_k256"].scaled(N=1, H=13, W=17),
    WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=17, W=15),
    WORKLOADS["conv7x7_c64_k64"].scaled(N=1, H=13, W=11),
    WORKLOADS["stem3x3s2_k16"].scaled(N=2, H=40, W=36),
    Workload("act_rw_c16", 80, 2, 11, 9, 16, 48, 1, 1, 1, 0, "f16"),
    Workload("act_narrow_c8_k24", 81, 2, 20, 18, 8, 24, 3, 3, 1, 1, "f16"),
    Workload("act_cout7", 82, 2, 9, 9, 16, 7, 3, 3, 2, 1, "f16"),
]


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("kernel", ["auto", "scalar", "igemm", "tiled"])
def test_act_shapes(act, kernel):
    ran = 0
    for wl in SHAPES:
        try:
            B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                         wl.dtype, kernel, act=act)
        except B.TgError:
            continue
        check_act(wl, act, kernel)
        ran += 1
    assert ran >= 2


# Kernel variants the dispatcher does not pick for these shapes, each through
# its switch (same switches as test_variants_gpu).
VARIANTS = [
    ({"cu": "0"}, WORKLOADS["conv1x1_c64_k256"].scaled(N=1, H=13, W=17), "igemm_rw"),
    ({"cu": "0", "igemm_rw": "0", "igemm_patch": "0"},
     WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=17, W=15), "igemm_dma"),
    ({"cu": "0", "igemm_rw": "0", "igemm_patch": "0", "igemm_dma": "0"},
     WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=17, W=15), "igemm"),
    ({"stem": "0"}, WORKLOADS["stem3x3s2_k16"].scaled(N=2, H=40, W=40), "tiled_mfma_pipe"),
    ({"stem": "0", "tm_pipe": "0"}, WORKLOADS["stem3x3s2_k16"].scaled(N=2, H=40, W=36),
     "tiled_mfma"),
    ({"stem": "0", "tiled_mfma": "0"},
     WORKLOADS["stem3x3s2_k16"].scaled(N=2, H=40, W=36), "tiled"),
]


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("env,wl,prefix", VARIANTS, ids=[v[2] for v in VARIANTS])
def test_act_variants(tune, act, env, wl, prefix):
    tune(**env)
    plan = check_act(wl, act)
    assert plan.describe().startswith(prefix), plan.describe()


@pytest.mark.parametrize("act", ["relu", "gelu", "none"])
@pytest.mark.parametrize("name", ["conv1x1_c64_k256", "conv3x3_c128_k128", "stem3x3s2_k16",
                                  "stem3x3s2_k24", "conv7x7_c64_k64"])
def test_act_full_size(name, act):
    """Full-size workloads in the dispatched configuration, every output
    against the oracle's conv_bn_act."""
    wl = WORKLOADS[name]
    d, plan, y = run_act(wl, act)
    ref = oracle.conv_bn_act(d["x"], d["w"], d["gamma"], d["beta"], d["mean"], d["var"],
                             float(d["eps"]), wl.stride, wl.pad, act)
    compare(y.cpu().numpy(), ref, wl.dtype, "%s/%s full" % (name, act))


def test_act_rejected_where_unsupported():
    wl = WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=8, W=8)
    for kernel in ("unfused", "split"):
        with pytest.raises(B.TgError):
            B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                         wl.dtype, kernel, act="gelu")
    d = make_inputs(wl)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items() if k != "eps"}
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype, act="relu")
    with pytest.raises(B.TgError):
        plan.run_train(t["x"], t["w"], t["gamma"], t["beta"])
