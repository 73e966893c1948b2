"""Helpers for the GPU parity tests: upload seeded inputs, run one plan through
the C ABI, and compare against the fp64 oracle.

Pass criterion per element (and no NaN anywhere):
  fp16 output: |gpu - oracle| <= 1e-2 * max(1, |oracle|)
  fp32 output: |gpu - oracle| <= 1e-4 * max(1, |oracle|)
Tighter bounds derived from the arithmetic are asserted as well: fp16 output
rounding contributes at most 2^-11 relative, fp32 accumulation of fp16
products and the hardware exp2/reciprocal add ~1e-6, so fp16 results must lie
within 2e-3 * max(1, |oracle|) and fp32 results within 1e-5 * max(1, |oracle|).
Every output element is compared, at the full workload sizes too.
"""
from __future__ import annotations

import collections
import sys

import numpy as np

import oracle
from conv2d_batchnorm_silu_amd import binding as B
from conv2d_batchnorm_silu_amd.inputs import make_inputs

TOL = {"f16": 1e-2, "f32": 1e-4}
TIGHT = {"f16": 2e-3, "f32": 1e-5}


def note(msg: str):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def to_device(d: dict):
    import torch
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in d.items() if k != "eps"}
    t["eps"] = float(d["eps"])
    return t


def fold(t):
    return B.bn_fold(t["gamma"], t["beta"], t["mean"], t["var"], t["eps"])


def run_plan(wl, t, kernel="auto", table=B.Table.MI355X, scale_bias=None, out=None):
    import torch
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype, kernel, table)
    note("%s kernel=%s plan=%s" % (wl.name, kernel, plan.describe()))
    scale, bias = scale_bias if scale_bias is not None else fold(t)
    y = plan.run(t["x"], t["w"], scale, bias, out=out)
    torch.cuda.synchronize()
    return plan, y


def compare(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    got = got.astype(np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert not np.isnan(got).any(), "%s: NaN in GPU output" % what
    scaled = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    worst = float(scaled.max()) if scaled.size else 0.0
    nviol = int((scaled > TOL[dtype]).sum())
    note("%s: n=%d max|err|=%.3g max scaled=%.3g violations=%d" % (
        what, got.size, float(np.abs(got - ref).max()) if got.size else 0.0, worst, nviol))
    assert nviol == 0, "%s: %d elements beyond %g (worst %.3g)" % (what, nviol, TOL[dtype], worst)
    assert worst <= TIGHT[dtype], "%s: worst scaled error %.3g beyond derived bound %g" % (
        what, worst, TIGHT[dtype])
    return worst


# Oracle results of full workloads, kept for the other kernels and variants
# a test module compares on the same inputs (a few hundred MB at most).
_ORACLE_CACHE: "collections.OrderedDict" = collections.OrderedDict()
_ORACLE_CACHE_MAX = 6


def oracle_full(wl, d):
    """The fp64 oracle on every output of ``wl`` (inputs ``d`` from
    make_inputs(wl)); results are cached per workload."""
    key = (wl, "silu")
    hit = _ORACLE_CACHE.get(key)
    if hit is not None:
        _ORACLE_CACHE.move_to_end(key)
        return hit
    ref = oracle.conv_bn_silu(d["x"], d["w"], d["gamma"], d["beta"], d["mean"], d["var"],
                              float(d["eps"]), wl.stride, wl.pad)
    _ORACLE_CACHE[key] = ref
    while len(_ORACLE_CACHE) > _ORACLE_CACHE_MAX:
        _ORACLE_CACHE.popitem(last=False)
    return ref


def check_workload(wl, kernel, d=None, t=None):
    """Run ``kernel`` on ``wl`` and compare every output element with the
    fp64 oracle; returns the GPU result (numpy)."""
    d = d if d is not None else make_inputs(wl)
    t = t if t is not None else to_device(d)
    plan, y = run_plan(wl, t, kernel)
    got = y.cpu().numpy()
    compare(got, oracle_full(wl, d), wl.dtype, "%s/%s full" % (wl.name, kernel))
    return got
