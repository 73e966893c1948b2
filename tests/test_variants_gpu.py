"""GPU parity of every kernel variant that the dispatcher does not pick by
default for some shape, each selected through its tuning key
(tg_conv_bn_silu_create_tuned) and checked against the fp64 oracle:

  * the one-workgroup-per-CU 1x1 kernel (cu = wavefronts per 64-channel
    slice, cu_pd = input prefetch depth), over C_out = 64..256, ragged
    pixel tails, fewer blocks than compute units and the full headline layer;
  * the streaming 1x1 kernel with and without full-line input staging
    (stream, xdma = prefetch depth);
  * the register-weights kernel's non-default splits and plain stores;
  * the stem kernel (3-channel 3x3 stride-2 layers) over channel counts,
    image sizes, pixel tails and wave counts (stem), and with it switched
    off the band-staged MFMA kernel with and without its persistent
    pipeline (tm_pipe) and the VALU tiled kernel (tiled_mfma=0);
  * the patch-staged implicit GEMM for stride-1 layers with C_in % 64 == 0
    in every tile configuration (patch_cfg), including partial channel
    tiles, ragged pixel tails and channel counts it declines;
  * the direct-to-LDS implicit GEMM in every tile configuration
    (igemm_patch=0, dma_cfg) and the classic one (igemm_dma=0).
"""
import pytest

from conv2d_batchnorm_silu_amd import binding as B
from conv2d_batchnorm_silu_amd.inputs import WORKLOADS, Workload

from gpu_cases import check_workload, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.library()


def _plan(wl, kernel="igemm"):
    return B.ConvBnSilu(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        wl.dtype, kernel)


ONE_BY_ONE = [
    Workload("c64_k256_tail", 41, 1, 13, 17, 64, 256, 1, 1, 1, 0, "f16"),
    Workload("c64_k64", 42, 2, 11, 9, 64, 64, 1, 1, 1, 0, "f16"),
    Workload("c64_k128", 43, 1, 21, 23, 64, 128, 1, 1, 1, 0, "f16"),
    Workload("c64_k192", 44, 3, 7, 5, 64, 192, 1, 1, 1, 0, "f16"),
    Workload("c64_k256_m9", 45, 1, 3, 3, 64, 256, 1, 1, 1, 0, "f16"),
    Workload("c64_k256_m16", 46, 1, 4, 4, 64, 256, 1, 1, 1, 0, "f16"),
    Workload("c64_k256_many", 47, 4, 40, 40, 64, 256, 1, 1, 1, 0, "f16",
             ("uniform", -3.0, 3.0)),
]

CU_CFGS = [("2", "1"), ("2", "2"), ("2", "3"), ("3", "2"), ("3", "3"), ("4", "1"), ("4", "2"),
           ("1", "2")]


@pytest.mark.parametrize("per_group,pd", CU_CFGS, ids=["r%s_pd%s" % c for c in CU_CFGS])
@pytest.mark.parametrize("wl", ONE_BY_ONE, ids=[w.name for w in ONE_BY_ONE])
def test_cu_kernel(tune, wl, per_group, pd):
    tune(cu=per_group)
    tune(cu_pd=pd)
    assert "igemm_cu" in _plan(wl).describe()
    check_workload(wl, "igemm")
    check_workload(wl, "unfused")


@pytest.mark.parametrize("per_group,pd", [("2", "2"), ("3", "2"), ("3", "3"), ("4", "1"),
                                          ("4", "2")])
def test_cu_kernel_headline(tune, per_group, pd):
    tune(cu=per_group)
    tune(cu_pd=pd)
    wl = WORKLOADS["conv1x1_c64_k256"]
    assert "igemm_cu" in _plan(wl, "auto").describe()
    check_workload(wl, "auto")


def test_cu_kernel_not_for_other_shapes(tune):
    tune(cu="2")
    for wl in (Workload("c32", 48, 1, 9, 9, 32, 256, 1, 1, 1, 0, "f16"),
               Workload("k96", 49, 1, 9, 9, 64, 96, 1, 1, 1, 0, "f16"),
               Workload("s2", 50, 1, 9, 9, 64, 256, 1, 1, 2, 0, "f16")):
        note("%s -> %s" % (wl.name, _plan(wl).describe()))
        assert "igemm_cu" not in _plan(wl).describe()
        check_workload(wl, "igemm")


@pytest.mark.parametrize("env", [
    {"stream": "8"},
    {"stream": "8", "xdma": "1"},
    {"stream": "8", "xdma": "2"},
    {"stream": "12", "xdma": "4"},
    {"stream": "8", "nt": "0"},
], ids=lambda e: "_".join("%s%s" % (k, v) for k, v in e.items()))
def test_stream_kernel(tune, env):
    tune(cu="0")
    tune(**env)
    for wl in ONE_BY_ONE[:4] + [Workload("c32_k96", 51, 2, 7, 9, 32, 96, 1, 1, 1, 0, "f16")]:
        check_workload(wl, "igemm")


@pytest.mark.parametrize("env", [
    {"rw_nf": "8", "rw_cs": "2", "rw_ncw": "4"},
    {"rw_nf": "4", "rw_cs": "1", "rw_ncw": "4"},
    {"nt": "0"},
    {"rw_wg_per_cu": "2"},
], ids=lambda e: "_".join("%s%s" % (k, v) for k, v in e.items()))
def test_register_weights_kernel(tune, env):
    tune(cu="0")
    tune(**env)
    for wl in ONE_BY_ONE[:4] + [Workload("c8_2x2", 52, 1, 9, 11, 8, 40, 2, 2, 1, 0, "f16")]:
        assert "igemm_rw" in _plan(wl).describe()
        check_workload(wl, "igemm")


def test_cu_kernel_falls_back_for_unaligned_batchnorm_vectors():
    """The one-workgroup-per-CU kernel fetches scale and bias with 16-byte
    loads; with vectors offset by one float the register-weights kernel runs."""
    wl = ONE_BY_ONE[0]
    from gpu_cases import compare, fold, oracle_full, to_device
    from conv2d_batchnorm_silu_amd.inputs import make_inputs
    d = make_inputs(wl)
    t = to_device(d)
    s, b = fold(t)
    sbuf = torch.empty(wl.C_out + 1, dtype=torch.float32, device="cuda")
    bbuf = torch.empty(wl.C_out + 1, dtype=torch.float32, device="cuda")
    sbuf[1:].copy_(s)
    bbuf[1:].copy_(b)
    plan = _plan(wl)
    assert "igemm_cu" in plan.describe()
    note("unaligned BN vectors: %s" % plan.describe())
    y = plan.run(t["x"], t["w"], sbuf[1:], bbuf[1:])
    torch.cuda.synchronize()
    compare(y.cpu().numpy(), oracle_full(wl, d), "f16", "cu fallback, unaligned scale/bias")


@pytest.mark.parametrize("env", [{"tm_pipe": "0"}, {"tm_pipe": "0", "tm_rows": "4"},
                                 {"tm_rows": "4"}, {"tiled_mfma": "0"}],
                         ids=["nopipe", "nopipe_r4", "pipe_r4", "valu"])
def test_tiled_variants(tune, env):
    tune(stem="0")
    tune(**env)
    for wl in (WORKLOADS["stem3x3s2_k16"].scaled(N=2), WORKLOADS["stem3x3s2_k24"].scaled(N=1),
               Workload("stem_odd", 53, 1, 37, 29, 3, 24, 3, 3, 2, 1, "f16")):
        check_workload(wl, "tiled")


STEM_SHAPES = [
    Workload("stem_k16_small", 60, 2, 40, 36, 3, 16, 3, 3, 2, 1, "f16"),
    Workload("stem_k24_odd_h", 61, 1, 37, 34, 3, 24, 3, 3, 2, 1, "f16"),
    Workload("stem_k8_q16", 62, 3, 32, 32, 3, 8, 3, 3, 2, 1, "f16"),
    Workload("stem_k32", 63, 1, 50, 48, 3, 32, 3, 3, 2, 1, "f16", ("uniform", -2.0, 2.0)),
    Workload("stem_k48_h2", 64, 2, 2, 64, 3, 48, 3, 3, 2, 1, "f16"),
    Workload("stem_k64", 65, 1, 34, 40, 3, 64, 3, 3, 2, 1, "f16"),
    Workload("stem_k16_tail", 66, 1, 33, 38, 3, 16, 3, 3, 2, 1, "f16"),
    # Many short bands per workgroup.
    Workload("stem_ring", 67, 96, 130, 16, 3, 16, 3, 3, 2, 1, "f16"),
]


@pytest.mark.parametrize("wpc,rows", [("3", ""), ("4", "1"), ("2", "2"), ("1", "")])
def test_stem_kernel(tune, wpc, rows):
    """Workgroups per CU and band heights: with one-row bands the full-size
    workloads give each workgroup many bands, so its three band buffers are
    refilled while its compute waves work."""
    tune(stem=wpc)
    tune(stem_rows=rows)
    for wl in STEM_SHAPES:
        d = _plan(wl, "tiled").describe()
        note("%s -> %s" % (wl.name, d))
        assert d.startswith("stem")
        check_workload(wl, "tiled")
        check_workload(wl, "unfused")
    for name in ("stem3x3s2_k16", "stem3x3s2_k24"):
        d = _plan(WORKLOADS[name], "auto").describe()
        note("%s -> %s" % (name, d))
        assert d.startswith("stem")
        check_workload(WORKLOADS[name], "auto")


PATCH_SHAPES = [
    WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=17, W=15),
    WORKLOADS["conv7x7_c64_k64"].scaled(N=1, H=13, W=11),
    Workload("p3x3_c64_k33", 54, 2, 12, 12, 64, 33, 3, 3, 1, 1, "f16"),
    Workload("p5x5_c256_k96", 55, 1, 9, 10, 256, 96, 5, 5, 1, 2, "f16"),
    Workload("p3x3_c64_k128_wide", 56, 1, 6, 70, 64, 128, 3, 3, 1, 1, "f16"),
    Workload("p1x1_pad_c64_k64", 57, 2, 9, 9, 64, 64, 1, 1, 1, 0, "f16"),
    Workload("p3x3_c192_k64", 58, 1, 8, 8, 192, 64, 3, 3, 1, 1, "f16"),
]


@pytest.mark.parametrize("cfg", [str(i) for i in range(10)])
def test_patch_kernel(tune, cfg):
    tune(cu="0")
    tune(igemm_rw="0")
    tune(patch_cfg=cfg)
    ran = 0
    for wl in PATCH_SHAPES:
        d = _plan(wl).describe()
        note("%s -> %s" % (wl.name, d))
        ran += "igemm_patch" in d
        check_workload(wl, "igemm")
        check_workload(wl, "unfused")
    assert ran >= 5


@pytest.mark.parametrize("cfg", [str(i) for i in range(11)])
def test_dma_kernel(tune, cfg):
    tune(cu="0")
    tune(igemm_rw="0")
    tune(igemm_patch="0")
    tune(dma_cfg=cfg)
    for wl in PATCH_SHAPES[:4] + [Workload("s2_c64", 59, 1, 15, 13, 64, 80, 3, 3, 2, 1, "f16")]:
        assert "igemm_dma" in _plan(wl).describe()
        check_workload(wl, "igemm")


@pytest.mark.parametrize("env", [{"igemm_rw": "0", "igemm_patch": "0"},
                                 {"igemm_rw": "0", "igemm_patch": "0", "igemm_dma": "0"}],
                         ids=["dma", "classic"])
def test_igemm_variants(tune, env):
    tune(cu="0")
    tune(**env)
    for wl in (WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=17, W=15),
               WORKLOADS["conv7x7_c64_k64"].scaled(N=1, H=13, W=11),
               ONE_BY_ONE[0], ONE_BY_ONE[2]):
        check_workload(wl, "igemm")


BAND_SHAPES = [
    WORKLOADS["conv3x3_c128_k128"].scaled(N=2),
    WORKLOADS["conv7x7_c64_k64"].scaled(N=1),
    WORKLOADS["conv3x3_c128_k128"].scaled(N=1, H=17, W=15),
    WORKLOADS["conv7x7_c64_k64"].scaled(N=2, H=13, W=11),
    Workload("b5x5_c64_k128", 70, 2, 9, 10, 64, 128, 5, 5, 1, 2, "f16"),
    Workload("b3x3_c64_k128_wide", 71, 1, 6, 70, 64, 128, 3, 3, 1, 1, "f16"),
    Workload("b3x3_c192_k64", 72, 2, 8, 8, 192, 64, 3, 3, 1, 1, "f16"),
    Workload("b1x1_c128_k64", 73, 3, 7, 9, 128, 64, 1, 1, 1, 0, "f16"),
    Workload("b3x3_nopad_c64_k64", 74, 3, 9, 30, 64, 64, 3, 3, 1, 0, "f16"),
    Workload("b1px_c128_k128", 75, 1, 1, 1, 128, 128, 3, 3, 1, 1, "f16"),
    Workload("b3x3_c192_k128_tail", 76, 2, 11, 13, 192, 128, 3, 3, 1, 1, "f16",
             ("uniform", -2.0, 2.0)),
]


@pytest.mark.parametrize("wl", BAND_SHAPES, ids=[w.name for w in BAND_SHAPES])
def test_band_kernel(tune, wl):
    """The band implicit GEMM (opt-in, band=1; stride-1 layers with C_in % 64
    == 0 and C_out 64 or 128): every output against the oracle, fused and as
    the first kernel of the unfused and split forms, including odd K-step
    counts (the zero-filter step past the last chunk) and one-pixel images."""
    tune(band=1)
    d = _plan(wl, "auto").describe()
    note("%s -> %s" % (wl.name, d))
    assert d.startswith("igemm_band"), d
    check_workload(wl, "auto")
    check_workload(wl, "unfused")
    check_workload(wl, "split")


def test_band_declines_other_shapes(tune):
    tune(band=1)
    for wl in (Workload("s2", 77, 1, 12, 12, 64, 128, 3, 3, 2, 1, "f16"),
               Workload("k96", 78, 1, 12, 12, 64, 96, 3, 3, 1, 1, "f16"),
               Workload("c32", 79, 1, 12, 12, 32, 64, 3, 3, 1, 1, "f16")):
        d = _plan(wl, "auto").describe()
        note("%s -> %s" % (wl.name, d))
        assert not d.startswith("igemm_band"), d
