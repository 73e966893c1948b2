"""GPU parity: every kernel behind the C ABI against the fp64 oracle.

Covers the six workloads at full size (every output element against the
oracle), a random sweep of small shapes that span
several tiles with ragged tails, the degenerate and edge shapes, the
BatchNorm fold, fused vs unfused agreement, guard canaries around y, the
misaligned-pointer fallback and a non-default stream.
"""
import numpy as np
import pytest

from conv2d_batchnorm_silu_amd import binding as B
from conv2d_batchnorm_silu_amd.inputs import WORKLOADS, Workload, make_inputs, random_small_workloads

from gpu_cases import (compare, check_workload, fold, note, oracle_full, run_plan, to_device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.library()


def _serves(wl, kernel):
    try:
        B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                     wl.dtype, kernel)
        return True
    except B.TgError:
        return False


def test_bn_fold_matches_definition():
    rng = np.random.default_rng(0)
    C = 300
    g = rng.uniform(0.5, 1.5, C).astype(np.float32)
    b = rng.normal(0, 0.3, C).astype(np.float32)
    m = rng.normal(0, 0.3, C).astype(np.float32)
    v = rng.uniform(0.5, 2.0, C).astype(np.float32)
    eps = np.float32(1e-5)
    dev = [torch.from_numpy(a).cuda() for a in (g, b, m, v)]
    note("bn_fold C=%d" % C)
    s, bi = B.bn_fold(*dev, float(eps))
    torch.cuda.synchronize()
    g64, b64, m64, v64 = (a.astype(np.float64) for a in (g, b, m, v))
    s_ref = g64 / np.sqrt(v64 + np.float64(eps))
    np.testing.assert_allclose(s.cpu().numpy(), s_ref, rtol=3e-7, atol=0)
    np.testing.assert_allclose(bi.cpu().numpy(), b64 - m64 * s_ref, rtol=0, atol=3e-7)


KERNELS = ["auto", "scalar", "tiled", "igemm", "unfused", "split"]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload(name, kernel):
    wl = WORKLOADS[name]
    if not _serves(wl, kernel):
        pytest.skip("%s does not serve %s" % (kernel, name))
    check_workload(wl, kernel)


SMALL = random_small_workloads(40, seed=123)


@pytest.mark.parametrize("kernel", ["scalar", "tiled", "igemm", "unfused", "split"])
def test_random_small_shapes(kernel):
    ran = 0
    for wl in SMALL:
        if kernel == "igemm" and wl.C_in % 8:
            wl = wl.scaled(C_in=8 * max(1, wl.C_in // 8))
        if not _serves(wl, kernel):
            continue
        check_workload(wl, kernel)
        ran += 1
    assert ran >= 10


EDGE = [
    Workload("single_pixel_pad", 11, 1, 1, 1, 8, 16, 3, 3, 1, 1, "f16"),
    Workload("window_equals_image", 12, 2, 5, 7, 8, 24, 5, 7, 1, 0, "f16"),
    Workload("stride3_pad2", 13, 3, 17, 13, 16, 33, 3, 3, 3, 2, "f16"),
    Workload("cout1", 14, 2, 9, 9, 8, 1, 3, 3, 1, 1, "f16"),
    Workload("cout7", 15, 2, 9, 9, 16, 7, 3, 3, 2, 1, "f16"),
    Workload("cout17", 16, 2, 12, 12, 8, 17, 1, 1, 1, 0, "f16"),
    Workload("cout31", 17, 1, 10, 10, 24, 31, 3, 3, 1, 1, "f16"),
    Workload("cout33", 18, 1, 10, 10, 24, 33, 3, 3, 1, 1, "f16"),
    Workload("cin3_k5", 19, 2, 19, 21, 3, 16, 5, 5, 2, 2, "f16", ("uniform", -1.0, 1.0)),
    Workload("m_tail_1x1", 20, 1, 13, 17, 64, 256, 1, 1, 1, 0, "f16"),
    Workload("k_tail_c8_3x3", 21, 2, 11, 9, 8, 64, 3, 3, 1, 1, "f16"),
    Workload("wide_cout_320", 22, 1, 6, 6, 16, 320, 1, 1, 1, 0, "f16"),
    Workload("pad_gt_half_k", 23, 1, 6, 6, 8, 16, 3, 3, 1, 3, "f16"),
    Workload("asym_window_f32", 24, 2, 8, 9, 3, 5, 2, 3, 2, 1, "f32"),
    Workload("large_values", 25, 1, 8, 8, 16, 32, 3, 3, 1, 1, "f16", ("normal", 400.0)),
]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("wl", EDGE, ids=[w.name for w in EDGE])
def test_edge_shapes(wl, kernel):
    if not _serves(wl, kernel):
        pytest.skip("%s does not serve %s" % (kernel, wl.name))
    check_workload(wl, kernel)


@pytest.mark.parametrize("name", ["conv1x1_c64_k256", "conv3x3_c128_k128", "stem3x3s2_k24",
                                  "conv7x7_c64_k64"])
def test_fused_matches_gpu_unfused_and_scalar(name):
    """Full-size cross-check of every output: the dispatched fused kernel
    against the unfused three-kernel baseline (same conv mainloop; differs only
    by fp16 rounding of t1 and t2), the split two-kernel form (rounding of t1)
    and the scalar kernel."""
    wl = WORKLOADS[name]
    d = make_inputs(wl)
    t = to_device(d)
    sb = fold(t)
    _, y = run_plan(wl, t, "auto", scale_bias=sb)
    _, yu = run_plan(wl, t, "unfused", scale_bias=sb)
    _, ysp = run_plan(wl, t, "split", scale_bias=sb)
    _, ys = run_plan(wl, t, "scalar", scale_bias=sb)
    yf = y.float()
    for other, what in ((yu.float(), "unfused"), (ysp.float(), "split"), (ys.float(), "scalar")):
        err = ((yf - other).abs() / other.abs().clamp(min=1.0)).max().item()
        note("%s fused vs %s: max scaled diff %.3g" % (name, what, err))
        assert err <= 1e-2
    assert not torch.isnan(yf).any()


@pytest.mark.parametrize("kernel", ["scalar", "tiled", "igemm"])
def test_guard_canaries(kernel):
    wl = Workload("guard", 31, 2, 10, 11, 16, 24, 3, 3, 1, 1, "f16")
    if not _serves(wl, kernel):
        pytest.skip("not served")
    d = make_inputs(wl)
    t = to_device(d)
    n = wl.N * wl.P * wl.Q * wl.C_out
    guard = 4096
    buf = torch.full((n + 2 * guard,), 12345.0, dtype=torch.float16, device="cuda")
    out = buf[guard:guard + n].view(wl.y_shape)
    run_plan(wl, t, kernel, out=out)
    assert (buf[:guard] == 12345.0).all() and (buf[guard + n:] == 12345.0).all()
    compare(out.cpu().numpy(), oracle_full(wl, d), "f16", "guard/%s" % kernel)


def test_misaligned_auto_falls_back_to_scalar():
    wl = WORKLOADS["conv1x1_c64_k256"].scaled(N=1, H=9, W=9)
    d = make_inputs(wl)
    t = to_device(d)
    xbuf = torch.empty(t["x"].numel() + 1, dtype=torch.float16, device="cuda")
    xmis = xbuf[1:].view(t["x"].shape)
    xmis.copy_(t["x"])
    t["x"] = xmis
    plan, y = run_plan(wl, t, "auto")
    assert plan.kernel == B.Kernel.IGEMM
    compare(y.cpu().numpy(), oracle_full(wl, d), "f16", "misaligned auto")
    forced = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, 1, 1, 1, 0, "f16", "igemm")
    s, b = fold(t)
    with pytest.raises(B.TgError) as e:
        forced.run(t["x"], t["w"], s, b)
    assert e.value.status == 3


def test_side_stream():
    wl = WORKLOADS["stem3x3s2_k16"].scaled(N=2)
    d = make_inputs(wl)
    t = to_device(d)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        plan = B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                            "f16", "auto")
        s, b = fold(t)
        y = plan.run(t["x"], t["w"], s, b)
    st.synchronize()
    compare(y.cpu().numpy(), oracle_full(wl, d), "f16", "side stream")
