"""GPU checks of the layout conversions (tg_filter_oihw_to_ohwi,
tg_nchw_to_nhwc, tg_nhwc_to_nchw): pure permutations, so bit-exact against
numpy's transpose of the same values; and a PyTorch-layout caller's path
(OIHW filters converted once, NCHW x converted, fused conv, y back to NCHW)
against the oracle."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from conv2d_batchnorm_silu_amd import binding as B
from conv2d_batchnorm_silu_amd.inputs import WORKLOADS, make_inputs

from gpu_cases import compare, note

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SHAPES = [(1, 3, 224, 224), (2, 130, 7, 9), (3, 64, 1, 1), (1, 1, 65, 63), (2, 256, 8, 8),
          (1, 5, 3, 2)]


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_nchw_nhwc_round_trip_bit_exact(shape, dtype):
    rng = np.random.default_rng(sum(shape))
    a = rng.normal(size=shape).astype(dtype)
    t = torch.from_numpy(a).cuda()
    nhwc = B.nchw_to_nhwc(t)
    back = B.nhwc_to_nchw(nhwc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(nhwc.cpu().numpy(), a.transpose(0, 2, 3, 1))
    np.testing.assert_array_equal(back.cpu().numpy(), a)
    note("layout %s %s bit-exact" % (shape, np.dtype(dtype).name))


@pytest.mark.parametrize("shape", [(64, 3, 7, 7), (256, 64, 1, 1), (33, 17, 3, 5), (1, 1, 1, 1)])
def test_filter_oihw_to_ohwi_bit_exact(shape):
    rng = np.random.default_rng(7)
    w = rng.normal(size=shape).astype(np.float16)
    got = B.filter_oihw_to_ohwi(torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), w.transpose(0, 2, 3, 1))


@pytest.mark.parametrize("name", ["conv3x3_c128_k128", "stem3x3s2_k16"])
def test_pytorch_layout_caller(name):
    """OIHW filters converted once, NCHW x converted per call, the fused
    kernel, y converted back to NCHW: the oracle's NHWC result, permuted."""
    wl = WORKLOADS[name].scaled(N=2)
    d = make_inputs(wl)
    x_nchw = torch.from_numpy(np.ascontiguousarray(d["x"].transpose(0, 3, 1, 2))).cuda()
    w_oihw = torch.from_numpy(np.ascontiguousarray(d["w"].transpose(0, 3, 1, 2))).cuda()
    bn = [torch.from_numpy(d[k]).cuda() for k in ("gamma", "beta", "mean", "var")]
    scale, bias = B.bn_fold(*bn, float(d["eps"]))
    w = B.filter_oihw_to_ohwi(w_oihw)
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype)
    y = B.nhwc_to_nchw(plan.run(B.nchw_to_nhwc(x_nchw), w, scale, bias))
    torch.cuda.synchronize()
    ref = oracle.conv_bn_silu(d["x"], d["w"], d["gamma"], d["beta"], d["mean"], d["var"],
                              float(d["eps"]), wl.stride, wl.pad)
    compare(y.cpu().numpy(), ref.transpose(0, 3, 1, 2), wl.dtype, "%s NCHW caller" % name)
