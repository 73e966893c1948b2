"""GPU tests of the load-time filter pre-pack for the patch-staged implicit
GEMM (tg_conv_bn_silu_pack_filter, tg_conv_bn_silu_run_packed):

  * the packed bytes equal a numpy packing written from the layout that the
    header documents (per 64-channel chunk, block of 16 output channels and
    K-group: 16 rows of 128/WK bytes whose 16-byte pieces are XOR-swizzled),
    in every tile configuration (one and two K-groups, partial channel
    blocks, several channel tiles);
  * run_packed is bit-identical to run with the OHWI filter (the kernel's LDS
    contents, hence its arithmetic, are the same), at small shapes in every
    configuration and over every output of the full 3x3 and 7x7 layers in the
    launch configuration the benchmark times; it also agrees with the fp64
    oracle directly;
  * the other epilogue activations and the fp8 output take the same path;
  * a plan whose kernel takes no packed filter, a short buffer and misaligned
    pointers are rejected.
"""
import ctypes

import numpy as np
import pytest

from conv2d_batchnorm_silu_amd import binding as B
from conv2d_batchnorm_silu_amd.inputs import WORKLOADS, Workload, make_inputs

from gpu_cases import compare, fold, note, oracle_full, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _k_groups(plan) -> int:
    d = plan.describe()
    assert "igemm_patch" in d, d
    return int(d.split("waves=")[1].split("x")[0])


def pack_reference(w: np.ndarray, wk: int) -> np.ndarray:
    """The documented packed layout, from the OHWI fp16 filter: byte
    ((kc*NB + ob)*WK + kg)*(2048/WK) + rr*(128/WK) + s*16 holds the 8 channels
    w[16*ob + rr][64*kc + kg*(64/WK) + 8*(s ^ swz(rr)) ...], swz(rr) =
    (rr >> 1) & 3 for two K-groups and (rr >> 1) & 7 for one; rows past
    C_out are zero."""
    C_out = w.shape[0]
    K = w.size // C_out
    nk, NB, ppr = K // 64, (C_out + 15) // 16, 8 // wk
    rows = np.zeros((NB * 16, K), dtype=np.float16)
    rows[:C_out] = w.reshape(C_out, K)
    src = rows.reshape(NB, 16, nk, wk, ppr, 8)   # [ob][rr][kc][kg][piece][e]
    out = np.zeros((nk, NB, wk, 16, ppr, 8), dtype=np.float16)
    for rr in range(16):
        swz = (rr >> 1) & (3 if wk == 2 else 7)
        for s in range(ppr):
            out[:, :, :, rr, s, :] = src[:, rr, :, :, s ^ swz, :].transpose(1, 0, 2, 3)
    return out.reshape(-1)


def _bits(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def _check_packed(plan, t, sb):
    wk = _k_groups(plan)
    n = plan.packed_filter_bytes()
    wp = plan.pack_filter(t["w"])
    torch.cuda.synchronize()
    ref = pack_reference(t["w"].cpu().numpy(), wk)
    assert n == ref.size * 2
    assert np.array_equal(_bits(wp), ref.view(np.uint8)), "packed layout differs"
    y = plan.run(t["x"], t["w"], *sb)
    yp = plan.run_packed(t["x"], wp, *sb)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(yp), _bits(y)), "run_packed differs from run"
    return yp


PACK_SHAPES = [
    WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=17, W=15),
    WORKLOADS["conv7x7_c64_k64"].scaled(N=1, H=13, W=11),
    Workload("p3x3_c64_k33", 54, 2, 12, 12, 64, 33, 3, 3, 1, 1, "f16"),
    Workload("p5x5_c256_k96", 55, 1, 9, 10, 256, 96, 5, 5, 1, 2, "f16"),
    Workload("p3x3_c192_k200", 59, 1, 8, 8, 192, 200, 3, 3, 1, 1, "f16"),
]


@pytest.mark.parametrize("cfg", [str(i) for i in range(10)])
def test_pack_layout_and_bit_identity(tune, cfg):
    tune(cu="0")
    tune(igemm_rw="0")
    tune(patch_cfg=cfg)
    ran = 0
    for wl in PACK_SHAPES:
        plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride,
                            wl.pad, wl.dtype, "igemm")
        note("%s cfg=%s -> %s" % (wl.name, cfg, plan.describe()))
        if "igemm_patch" not in plan.describe():
            assert plan.packed_filter_bytes() == 0
            continue
        d = make_inputs(wl)
        t = to_device(d)
        yp = _check_packed(plan, t, fold(t))
        if ran == 0:
            compare(yp.cpu().numpy(), oracle_full(wl, d), wl.dtype, "%s packed" % wl.name)
        ran += 1
    assert ran >= 3


@pytest.mark.parametrize("name", ["conv3x3_c128_k128", "conv7x7_c64_k64"])
def test_pack_full_size(name):
    """Every output of the full layer, default plan (the one bench.py times)."""
    wl = WORKLOADS[name]
    d = make_inputs(wl)
    t = to_device(d)
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype, "auto")
    note("%s -> %s" % (name, plan.describe()))
    yp = _check_packed(plan, t, fold(t))
    compare(yp.cpu().numpy(), oracle_full(wl, d), wl.dtype, "%s packed full" % name)


@pytest.mark.parametrize("act,out_dtype", [("relu", None), ("gelu", None), ("none", None),
                                           ("silu", "f8")])
def test_pack_other_epilogues(act, out_dtype):
    wl = WORKLOADS["conv3x3_c128_k128"].scaled(N=2, H=14, W=14)
    t = to_device(make_inputs(wl))
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype, "auto", act=act, out_dtype=out_dtype)
    note("%s act=%s y=%s -> %s" % (wl.name, act, out_dtype, plan.describe()))
    _check_packed(plan, t, fold(t))


def test_pack_rejections():
    lib = B.library()
    wl = WORKLOADS["conv1x1_c64_k256"].scaled(N=1)
    one = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, 1, 1, 1, 0, "f16", "auto")
    assert one.packed_filter_bytes() == 0
    w1 = torch.zeros((wl.C_out, 1, 1, wl.C_in), dtype=torch.float16, device="cuda")
    with pytest.raises(B.TgError):
        one.pack_filter(w1)

    wl = WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=14, W=14)
    t = to_device(make_inputs(wl))
    plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, 3, 3, 1, 1, "f16", "auto")
    n = plan.packed_filter_bytes()
    buf = torch.zeros(n + 16, dtype=torch.uint8, device="cuda")
    st = lib.tg_conv_bn_silu_pack_filter(plan._h, t["w"].data_ptr(), buf.data_ptr(), n - 16,
                                         None)
    assert st == 4  # TG_ERR_WORKSPACE
    st = lib.tg_conv_bn_silu_pack_filter(plan._h, t["w"].data_ptr(), buf.data_ptr() + 8, n,
                                         None)
    assert st == 3  # TG_ERR_ALIGNMENT
    wp = plan.pack_filter(t["w"])
    sc, bi = fold(t)
    y = torch.empty(plan.y_shape, dtype=torch.float16, device="cuda")
    xb = torch.zeros(t["x"].numel() + 8, dtype=torch.float16, device="cuda")
    st = lib.tg_conv_bn_silu_run_packed(plan._h, xb.data_ptr() + 2, wp.data_ptr(),
                                        sc.data_ptr(), bi.data_ptr(), y.data_ptr(), None)
    assert st == 3  # TG_ERR_ALIGNMENT: no scalar fallback for a packed filter
    st = lib.tg_conv_bn_silu_run_packed(one._h, xb.data_ptr(), wp.data_ptr(), sc.data_ptr(),
                                        bi.data_ptr(), y.data_ptr(), None)
    assert st == 2  # TG_ERR_UNSUPPORTED
    torch.cuda.synchronize()
