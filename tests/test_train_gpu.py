"""GPU parity of training-mode BatchNorm (batch statistics) through the C ABI
(tg_conv_bn_silu_train_run) against the fp64 oracle's conv_bn_silu_train.

Bars (no NaN anywhere): y as for the inference path, |gpu - oracle| <=
1e-2 * max(1, |oracle|) for fp16 and 1e-4 * max(1, |oracle|) for fp32. A
tighter bound follows from the arithmetic: outside the 1x1 layer the conv
output t1 is stored in the plan's dtype before the statistics and the
normalisation read it, so for fp16 each normalised value carries t1's
rounding (2^-11 relative of |t1|) scaled by gamma/sigma, plus y's own
rounding; with the seeded data (|t1|/sigma below about 6, gamma <= 1.5) that
is below 5e-3 * max(1, |oracle|) (the 1x1 layer normalises the fp32
accumulators of a second conv pass and carries only y's rounding). The batch
mean and (biased) variance and the updated running estimates are fp32
results of fp64 sums over rounded t1 (over the fp32 accumulators for the 1x1
kernel, which forms them in a statistics-only pass): within
1e-3 * max(1, |oracle|) for fp16 and 1e-5 for fp32. The reductions combine
their partials in a fixed order, so two calls give bit-identical results.
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

Y_TOL = {"f16": 1e-2, "f32": 1e-4}
Y_TIGHT = {"f16": 5e-3, "f32": 1e-5}
STAT_TOL = {"f16": 1e-3, "f32": 1e-5}


def _scaled(got, ref):
    got = np.asarray(got, dtype=np.float64)
    return np.abs(got - ref) / np.maximum(1.0, np.abs(ref))


def run_train(wl, kernel="auto", momentum=0.1, d=None, w_override=None):
    d = d if d is not None else make_inputs(wl)
    if w_override is not None:
        d = dict(d, w=w_override)
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in d.items() if k != "eps"}
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype, kernel)
    note("%s train kernel=%s plan=%s" % (wl.name, kernel, plan.describe()))
    rm, rv = t["mean"].clone(), t["var"].clone()  # running estimates before the step
    y, bm, bv = plan.run_train(t["x"], t["w"], t["gamma"], t["beta"], float(d["eps"]), momentum,
                               rm, rv)
    torch.cuda.synchronize()
    ref = oracle.conv_bn_silu_train(d["x"], d["w"], d["gamma"], d["beta"], float(d["eps"]),
                                    wl.stride, wl.pad, d["mean"], d["var"], momentum)
    return d, (y, bm, bv, rm, rv), ref


def check(wl, kernel="auto", momentum=0.1):
    d, (y, bm, bv, rm, rv), ref = run_train(wl, kernel, momentum)
    got = y.float().cpu().numpy()
    assert not np.isnan(got).any()
    ey = float(_scaled(got, ref["y"]).max())
    stats = {"mean": bm, "var": bv, "running_mean": rm, "running_var": rv}
    es = {k: float(_scaled(v.cpu().numpy(), ref[k]).max()) for k, v in stats.items()}
    note("%s/%s: y max scaled error %.3g; stats %s" % (
        wl.name, kernel, ey, ", ".join("%s %.3g" % kv for kv in es.items())))
    assert ey <= Y_TOL[wl.dtype]
    assert ey <= Y_TIGHT[wl.dtype]
    for k, e in es.items():
        assert e <= STAT_TOL[wl.dtype], (k, e)


SHAPES = [
    WORKLOADS["tiny_f32_3x3"],
    WORKLOADS["conv3x3_c128_k128"].scaled(N=2, H=15, W=13),
    WORKLOADS["conv7x7_c64_k64"].scaled(N=1, H=12, W=11),
    WORKLOADS["stem3x3s2_k24"].scaled(N=2, H=34, W=30),
    Workload("train_1x1_c64_k256", 70, 2, 9, 11, 64, 256, 1, 1, 1, 0, "f16"),
    Workload("train_cout7", 71, 3, 10, 9, 16, 7, 3, 3, 2, 1, "f16"),
    Workload("train_cout33_f32", 72, 2, 7, 8, 5, 33, 3, 3, 1, 1, "f32", ("uniform", -1.0, 1.0)),
    Workload("train_m2", 73, 2, 1, 1, 8, 16, 1, 1, 1, 0, "f16"),
    Workload("train_large_values", 74, 2, 9, 9, 8, 16, 3, 3, 1, 1, "f16", ("normal", 30.0)),
    # more channels than the statistics block has lanes (640 > 512)
    Workload("train_wide_c640", 76, 2, 5, 6, 16, 640, 1, 1, 1, 0, "f16"),
    # the stem's statistics pass keeps 1, 3 and 4 channel blocks of 8; 40
    # channels take the t1 path
    Workload("train_stem_c8", 77, 3, 22, 18, 3, 8, 3, 3, 2, 1, "f16", ("uniform", -1.0, 1.0)),
    Workload("train_stem_c24_odd_h", 78, 2, 23, 30, 3, 24, 3, 3, 2, 1, "f16", ("uniform", -1.0, 1.0)),
    Workload("train_stem_c32", 79, 2, 20, 26, 3, 32, 3, 3, 2, 1, "f16", ("uniform", -1.0, 1.0)),
    Workload("train_stem_c40", 80, 2, 16, 16, 3, 40, 3, 3, 2, 1, "f16", ("uniform", -1.0, 1.0)),
]


@pytest.mark.parametrize("kernel", ["auto", "scalar", "igemm", "tiled"])
@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_train_small(wl, kernel):
    try:
        B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                     wl.dtype, kernel)
    except B.TgError:
        pytest.skip("%s does not serve %s" % (kernel, wl.name))
    check(wl, kernel)


@pytest.mark.parametrize("name", ["conv1x1_c64_k256", "conv3x3_c128_k128", "stem3x3s2_k16"])
def test_train_full_size(name):
    """Full-size workloads in the launch configuration of the fused path:
    every output, and the statistics over all M rows."""
    check(WORKLOADS[name], "auto", momentum=0.25)


def test_train_constant_channel():
    """A zero filter makes its channel's conv output 0 everywhere: variance 0,
    output silu(beta) for every pixel."""
    wl = Workload("train_const", 75, 2, 8, 8, 16, 32, 3, 3, 1, 1, "f16")
    d = make_inputs(wl)
    w = d["w"].copy()
    w[5] = 0
    _, (y, bm, bv, _, _), ref = run_train(wl, d=d, w_override=w)
    got = y.float().cpu().numpy()
    assert float(bv[5]) == 0.0 and float(bm[5]) == 0.0
    want = oracle.silu(np.float64(d["beta"][5]))
    assert np.abs(got[..., 5] - want).max() <= 1e-3 * max(1.0, abs(want))
    assert float(_scaled(got, ref["y"]).max()) <= Y_TIGHT["f16"]


@pytest.mark.parametrize("name", ["conv3x3_c128_k128", "conv1x1_c64_k256", "stem3x3s2_k24"])
def test_train_deterministic(name):
    """Two calls give identical y and batch statistics: the row-block sums
    (3x3) and the 1x1 and stem kernels' per-workgroup triples are merged in a
    fixed order whatever the scheduling."""
    wl = WORKLOADS[name].scaled(N=4)
    d = make_inputs(wl)
    outs = [run_train(wl, d=d)[1] for _ in range(2)]
    for a, b in zip(outs[0][:3], outs[1][:3]):
        assert torch.equal(a, b)


def test_train_statistics_large_offset():
    """Inputs around 30 with a spread of 0.6 make every channel's conv output
    mean some 50 standard deviations away from 0, where
    sum(x^2) - sum(x)^2/M would cancel. The 1x1 kernel forms its statistics
    from the fp32 accumulators (shifted, merged as count/mean/squared
    deviations): they match the oracle's exact batch statistics. The other
    kernels read the stored fp16 t1, whose rounding (2^-11 of |t1|, about a
    twentieth of sigma here) moves the variance itself: their statistics match
    those of the oracle's conv output rounded to fp16, up to the few stored
    values that sit one fp16 step (0.03 here) from that rounding because the
    fp32 sum ends on the other side of a rounding boundary: with 128 outputs
    per channel those move the variance by a few 1e-4. y carries t1's
    rounding too, so only the statistics are compared."""
    for wl, exact in ((Workload("train_offset_1x1", 77, 4, 14, 14, 64, 128, 1, 1, 1, 0, "f16",
                                ("uniform", 29.0, 31.0)), True),
                      (Workload("train_offset_3x3", 78, 2, 10, 10, 64, 64, 3, 3, 1, 0, "f16",
                                ("uniform", 29.0, 31.0)), False)):
        d, (y, bm, bv, rm, rv), ref = run_train(wl)
        assert not np.isnan(y.float().cpu().numpy()).any()
        assert np.median(np.abs(ref["mean"]) / np.sqrt(ref["var"])) > 10.0
        if exact:
            mean, var = ref["mean"], ref["var"]
        else:
            t = oracle.conv2d(d["x"], d["w"], wl.stride, wl.pad)
            flat = t.astype(np.float16).astype(np.float64).reshape(-1, wl.C_out)
            mean = flat.mean(axis=0)
            var = ((flat - mean) ** 2).mean(axis=0)
        e_mean = float(np.abs(bm.cpu().numpy() - mean).max() / np.abs(mean).max())
        e_var = float((np.abs(bv.cpu().numpy() - var) / var).max())
        note("%s: mean error %.3g (relative to max |mean|), variance relative error %.3g" % (
            wl.name, e_mean, e_var))
        if exact:
            assert e_mean <= 1e-6 and e_var <= 1e-5, (e_mean, e_var)
        else:
            assert e_mean <= 1e-5 and e_var <= 2e-3, (e_mean, e_var)


def test_train_no_running_update_and_errors():
    wl = WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=8, W=8)
    d = make_inputs(wl)
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in d.items() if k != "eps"}
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype)
    y, bm, bv = plan.run_train(t["x"], t["w"], t["gamma"], t["beta"])
    torch.cuda.synchronize()
    ref = oracle.conv_bn_silu_train(d["x"], d["w"], d["gamma"], d["beta"], 1e-5, 1, 1)
    assert float(_scaled(y.float().cpu().numpy(), ref["y"]).max()) <= Y_TIGHT["f16"]
    small = torch.empty(plan.train_workspace_bytes() - 256, dtype=torch.uint8, device=dev)
    with pytest.raises(B.TgError):
        plan.run_train(t["x"], t["w"], t["gamma"], t["beta"], workspace=small)
