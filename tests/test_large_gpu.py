"""The largest inputs the library accepts, on the GPU, against the oracle at
sampled outputs (the oracle's per-output entry; every output would take the
fp64 oracle minutes at these sizes).

* A 1x1 layer (64 -> 64 channels) whose x and y each hold 2.26 GB: byte
  offsets need more than 31 bits, so the fast 1x1 kernels (32-bit buffer
  offsets) decline and the plan falls back to the classic implicit GEMM.
* An RGB stem (3x3, stride 2) whose x holds 2.21 GB: the stem and band-staged
  MFMA kernels decline for the same reason, the VALU tiled kernel serves.
* An fp32 1x1 layer with 2^31 - 16 outputs, sixteen below the largest count
  create() accepts (2^31 - 1 elements): the scalar kernel's grid at the
  limit.

Samples: 4000 seeded random outputs, the first and last 64 and the corners of
the first and last image. Inputs come from the seeded generators of
conv2d_batchnorm_silu_amd.inputs. Tolerances as everywhere (1e-2 fp16, 1e-4
fp32, scaled by max(1, |oracle|), with the tighter derived bounds).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from conv2d_batchnorm_silu_amd import binding as B
from conv2d_batchnorm_silu_amd.inputs import Workload, make_inputs

from gpu_cases import compare, fold, note, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _samples(wl, n=4000, seed=5):
    total = wl.N * wl.P * wl.Q * wl.C_out
    rng = np.random.default_rng(seed)
    img = wl.P * wl.Q * wl.C_out
    fixed = np.concatenate([np.arange(64), total - 64 + np.arange(64),
                            [0, wl.C_out - 1, img - 1, img - wl.C_out,
                             total - img, total - 1]])
    return np.unique(np.concatenate([rng.integers(0, total, n), fixed])).astype(np.int64)


def _check(wl, expect_not=()):
    d = make_inputs(wl)
    t = to_device(d)
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype)
    desc = plan.describe()
    note("%s: %s" % (wl.name, desc))
    for k in expect_not:
        assert not desc.startswith(k), desc
    sc, bi = fold(t)
    y = plan.run(t["x"], t["w"], sc, bi)
    torch.cuda.synchronize()
    idx = _samples(wl)
    got = y.reshape(-1)[torch.from_numpy(idx).to(y.device)].cpu().numpy()
    del y
    torch.cuda.empty_cache()
    ref = oracle.conv_bn_silu_at(d["x"], d["w"], d["gamma"], d["beta"], d["mean"], d["var"],
                                 float(d["eps"]), wl.stride, wl.pad, idx)
    compare(got, ref, wl.dtype, "%s sampled" % wl.name)


def test_1x1_beyond_31_bit_offsets():
    wl = Workload("big_1x1", 90, 1, 4200, 4200, 64, 64, 1, 1, 1, 0, "f16")
    assert 2 * wl.N * wl.H * wl.W * wl.C_in > 2**31
    _check(wl, expect_not=("igemm_cu", "igemm_rw", "igemm_stream", "igemm_patch",
                           "igemm_dma"))


def test_stem_beyond_31_bit_offsets():
    wl = Workload("big_stem", 91, 16, 4800, 4800, 3, 16, 3, 3, 2, 1, "f16",
                  ("uniform", -1.0, 1.0))
    assert 2 * wl.N * wl.H * wl.W * wl.C_in > 2**31
    _check(wl, expect_not=("stem", "tiled_mfma"))


def test_fp32_outputs_at_the_element_limit():
    # 2^31 - 16 = 16 * 7 * 73 * 262657: 511 x 262657 pixels, 16 channels.
    wl = Workload("limit_f32", 92, 1, 511, 262657, 1, 16, 1, 1, 1, 0, "f32",
                  ("uniform", -1.0, 1.0))
    assert wl.N * wl.P * wl.Q * wl.C_out == 2**31 - 16
    _check(wl)
