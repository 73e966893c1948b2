"""tg_conv_bn_silu_train_run_static (workspace in the library's static
device array, nothing allocated) against tg_conv_bn_silu_train_run (the
caller's workspace), through the C ABI: two calls in a row on one GPU, the
second with a smaller input, every output compared. Both entry points run
the same kernels in the same fixed order, so y, the batch statistics and the
updated running estimates must agree bit for bit (a stricter bar than the
oracle tolerance, which the training tests already check for run_train).
A plan whose workspace exceeds the static array is rejected before any
launch."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from conv2d_batchnorm_silu_amd import binding as B
from conv2d_batchnorm_silu_amd.inputs import WORKLOADS, Workload, make_inputs

from gpu_cases import note

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

UNSUP = 2


def _pair(wl):
    d = make_inputs(wl)
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in d.items() if k != "eps"}
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype)
    note("%s: %s" % (wl.name, plan.describe()))
    eps, mom = float(d["eps"]), 0.2
    rm_a, rv_a = t["mean"].clone(), t["var"].clone()
    rm_b, rv_b = t["mean"].clone(), t["var"].clone()
    ya, bma, bva = plan.run_train(t["x"], t["w"], t["gamma"], t["beta"], eps, mom, rm_a, rv_a)
    torch.cuda.synchronize()
    # Static entry, outputs preallocated: the call itself allocates nothing.
    yb = torch.full_like(ya, float("nan"))
    bmb = torch.full_like(bma, float("nan"))
    bvb = torch.full_like(bva, float("nan"))
    plan.run_train_static(t["x"], t["w"], t["gamma"], t["beta"], eps, mom, rm_b, rv_b,
                          out=yb, batch_mean=bmb, batch_var=bvb)
    torch.cuda.synchronize()
    for name, a, b in (("y", ya, yb), ("batch_mean", bma, bmb), ("batch_var", bva, bvb),
                       ("running_mean", rm_a, rm_b), ("running_var", rv_a, rv_b)):
        assert not torch.isnan(b).any(), name
        assert torch.equal(a, b), (wl.name, name,
                                   float((a.float() - b.float()).abs().max()))
    note("%s: static entry equals run_train on every output" % wl.name)


def test_static_entry_matches_train_run_twice():
    """The full 1x1 layer (statistics in the conv epilogue), then a smaller
    3x3 layer (statistics pass): the second call reuses the array the first
    one filled."""
    _pair(WORKLOADS["conv1x1_c64_k256"])
    _pair(Workload("static_small_3x3", 81, 2, 12, 10, 64, 64, 3, 3, 1, 1, "f16"))


def test_static_entry_rejects_oversized_plans():
    """1024 channels over 512 row blocks need 8 MiB of partials."""
    lib = B.library()
    plan = B.ConvBnSilu(64, 56, 56, 64, 1024, 1, 1, 1, 0, "f16")
    assert plan.train_workspace_bytes() > 4 << 20
    a = 1 << 20  # never dereferenced: the size check comes first
    st = lib.tg_conv_bn_silu_train_run_static(plan._h, a, a, a, a, 1e-5, 0.1, None, None, None,
                                              None, a, None)
    assert st == UNSUP
