"""The C ABI under HIP graph capture: tg_conv_bn_silu_run (fused, split) and
tg_conv_bn_silu_train_run launch only kernels on the caller's stream (no
memset, no allocation, no synchronisation), so a caller can capture them into
a graph and replay it. Each graph is replayed several times with eager work
and synchronisations in between, and every replay must equal the eager
result bit for bit (same kernels, same inputs)."""
from __future__ import annotations

import numpy as np
import pytest

from conv2d_batchnorm_silu_amd import binding as B
from conv2d_batchnorm_silu_amd.inputs import WORKLOADS, make_inputs

from gpu_cases import note

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [("conv1x1_c64_k256", "auto"), ("conv3x3_c128_k128", "auto"),
         ("stem3x3s2_k16", "auto"), ("conv3x3_c128_k128", "split")]


def _setup(name, N=4):
    wl = WORKLOADS[name].scaled(N=N)
    d = make_inputs(wl)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items() if k != "eps"}
    return wl, d, t


@pytest.mark.parametrize("name,kernel", CASES, ids=["%s-%s" % c for c in CASES])
def test_graph_replay_matches_eager(name, kernel):
    wl, d, t = _setup(name)
    scale, bias = B.bn_fold(t["gamma"], t["beta"], t["mean"], t["var"], float(d["eps"]))
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype, kernel)
    note("graph %s %s" % (name, plan.describe()))
    ws = (torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
          if plan.workspace_bytes else None)
    ref = plan.run(t["x"], t["w"], scale, bias, workspace=ws)  # eager; sets kernel attributes
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        plan.run(t["x"], t["w"], scale, bias, out=out, workspace=ws)
    for i in range(3):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d differs from the eager result" % i
        del junk


def test_graph_replay_training_mode():
    wl, d, t = _setup("conv3x3_c128_k128")
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype)
    ws = torch.empty(plan.train_workspace_bytes(), dtype=torch.uint8, device="cuda")
    ref, rbm, rbv = plan.run_train(t["x"], t["w"], t["gamma"], t["beta"], workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    lib = plan._lib
    bm, bv = torch.empty_like(rbm), torch.empty_like(rbv)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st = lib.tg_conv_bn_silu_train_run(
            plan._h, t["x"].data_ptr(), t["w"].data_ptr(), t["gamma"].data_ptr(),
            t["beta"].data_ptr(), 1e-5, 0.1, None, None, bm.data_ptr(), bv.data_ptr(),
            out.data_ptr(), ws.data_ptr(), ws.numel(), s.cuda_stream)
        assert st == 0
    for i in range(3):
        out.fill_(float("nan"))
        bm.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(bm, rbm) and torch.equal(bv, rbv), i
