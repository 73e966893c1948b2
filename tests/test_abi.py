"""The C ABI on the host: the library loads, exports every function the
header declares, validates its arguments and makes its dispatch decisions --
all without touching a GPU (no call here reaches a kernel launch)."""
import ctypes

import pytest

from conv2d_batchnorm_silu_amd import binding as B
from conv2d_batchnorm_silu_amd.inputs import WORKLOADS

OK, INVAL, UNSUP, ALIGN, WS, HIPERR = range(6)


@pytest.fixture(scope="module")
def lib():
    return B.library()


def _create(lib, *shape, dtype=0, kernel=0, table=0):
    h = ctypes.c_void_p()
    st = lib.tg_conv_bn_silu_create_with_table(ctypes.byref(h), *shape, dtype, kernel, table)
    return st, h


def test_exports_every_declared_symbol(lib):
    names = B.exported_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert "tg_conv_bn_silu_create" in names and "tg_bn_fold" in names


@pytest.mark.parametrize("bad", [
    (0, 8, 8, 3, 4, 3, 3, 1, 1), (1, 0, 8, 3, 4, 3, 3, 1, 1), (1, 8, 8, 0, 4, 3, 3, 1, 1),
    (1, 8, 8, 3, 0, 3, 3, 1, 1), (1, 8, 8, 3, 4, 0, 3, 1, 1), (1, 8, 8, 3, 4, 3, 3, 0, 1),
    (1, 8, 8, 3, 4, 3, 3, 1, -1), (1, 2, 8, 3, 4, 5, 3, 1, 1), (1, 8, 1, 3, 4, 3, 3, 1, 0)])
def test_create_rejects_invalid(lib, bad):
    st, h = _create(lib, *bad)
    assert st == INVAL and not h.value


def test_create_null_out(lib):
    assert lib.tg_conv_bn_silu_create(None, 1, 8, 8, 3, 4, 3, 3, 1, 1, 0, 0) == INVAL


def test_create_unsupported(lib):
    # 2^31 output elements
    assert _create(lib, 2048, 1024, 1024, 1, 1, 1, 1, 1, 0)[0] == UNSUP
    # unknown dtype, kernel, table
    assert _create(lib, 1, 8, 8, 8, 8, 3, 3, 1, 1, dtype=7)[0] == UNSUP
    assert _create(lib, 1, 8, 8, 8, 8, 3, 3, 1, 1, kernel=9)[0] == UNSUP
    assert _create(lib, 1, 8, 8, 8, 8, 3, 3, 1, 1, table=5)[0] == UNSUP
    # igemm needs fp16 and C_in % 8 == 0
    assert _create(lib, 1, 8, 8, 3, 8, 3, 3, 1, 1, kernel=3)[0] == UNSUP
    assert _create(lib, 1, 8, 8, 8, 8, 3, 3, 1, 1, dtype=1, kernel=3)[0] == UNSUP
    # tiled is fp16 only and needs C_out <= 64
    assert _create(lib, 1, 8, 8, 8, 8, 3, 3, 1, 1, dtype=1, kernel=2)[0] == UNSUP
    assert _create(lib, 1, 8, 8, 8, 65, 3, 3, 1, 1, kernel=2)[0] == UNSUP


def test_query_and_describe(lib):
    for wl in WORKLOADS.values():
        st, h = _create(lib, wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride, wl.pad,
                        dtype=0 if wl.dtype == "f16" else 1)
        assert st == OK
        P, Q, k, ws = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_size_t()
        assert lib.tg_conv_bn_silu_query(h, ctypes.byref(P), ctypes.byref(Q), ctypes.byref(k),
                                         ctypes.byref(ws)) == OK
        assert (P.value, Q.value) == (wl.P, wl.Q) and ws.value == 0
        assert k.value in (1, 2, 3)
        buf = ctypes.create_string_buffer(256)
        assert lib.tg_conv_bn_silu_describe(h, buf, 256) == OK
        assert ("%dx%d" % (wl.P, wl.Q)).encode() in buf.value
        assert lib.tg_conv_bn_silu_destroy(h) == OK
    assert lib.tg_conv_bn_silu_query(None, None, None, None, None) == INVAL
    assert lib.tg_conv_bn_silu_destroy(None) == OK


def test_unfused_workspace_size(lib):
    wl = WORKLOADS["conv1x1_c64_k256"]
    st, h = _create(lib, wl.N, wl.H, wl.W, wl.C_in, wl.C_out, 1, 1, 1, 0, kernel=0x100)
    assert st == OK
    k, ws = ctypes.c_int(), ctypes.c_size_t()
    lib.tg_conv_bn_silu_query(h, None, None, ctypes.byref(k), ctypes.byref(ws))
    ybytes = wl.N * wl.P * wl.Q * wl.C_out * 2
    assert ws.value == 2 * ((ybytes + 255) // 256 * 256)
    assert k.value == (3 | 0x100)
    lib.tg_conv_bn_silu_destroy(h)


def test_pages_dispatch_table():
    """The page's thresholds: GEMM for 1x1 with >= 32 output channels, tiled
    above 16 output channels, scalar otherwise (tiled only where it can serve
    the shape)."""
    want = {"tiny_f32_3x3": B.Kernel.SCALAR, "conv1x1_c64_k256": B.Kernel.IGEMM,
            "stem3x3s2_k16": B.Kernel.SCALAR, "stem3x3s2_k24": B.Kernel.TILED,
            # tiled holds the filter bank in LDS: 3x3x128 and 7x7x64 banks do not fit
            "conv3x3_c128_k128": B.Kernel.SCALAR, "conv7x7_c64_k64": B.Kernel.SCALAR}
    for name, k in want.items():
        wl = WORKLOADS[name]
        dt = B.Dtype.F16 if wl.dtype == "f16" else B.Dtype.F32
        got = B.dispatch_choose(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride,
                                wl.pad, dt, B.Table.PAGES)
        assert got == k, name
    # boundary cases of the thresholds
    ch = lambda co, k=1, ci=16: B.dispatch_choose(2, 16, 16, ci, co, k, k, 1, k // 2,
                                                  B.Dtype.F16, B.Table.PAGES)
    assert ch(32) == B.Kernel.IGEMM and ch(31) == B.Kernel.TILED
    assert ch(17) == B.Kernel.TILED and ch(16) == B.Kernel.SCALAR
    assert ch(32, k=3) == B.Kernel.TILED


def test_mi355x_dispatch_table_regions():
    """The MI355X table's measured regions (sweep over k, stride, C_in,
    C_out at 10^5 output pixels): implicit GEMM for C_in % 8 == 0 except
    1x1 layers with K < 32 and C_out <= 32 (MFMA tiled kernel); for RGB
    input tiled, except 1x1 layers past C_out 32 (scalar)."""
    ch = lambda ci, co, k=1, s=1: B.dispatch_choose(8, 112 * s, 112 * s, ci, co, k, k, s, k // 2,
                                                    B.Dtype.F16, B.Table.MI355X)
    for co in (8, 12, 16, 20, 24, 32):
        assert ch(16, co) == B.Kernel.TILED, co      # K = 16 < 32
    for co in (48, 64, 128, 256):
        assert ch(16, co) == B.Kernel.IGEMM, co
    for ci in (16, 64, 128):
        for co in (8, 12):
            for k in (3, 5, 7):
                assert ch(ci, co, k) == B.Kernel.IGEMM, (ci, co, k)
        assert ch(ci, 8, 1, 2) == (B.Kernel.TILED if ci == 16 else B.Kernel.IGEMM), ci
    for co in (8, 16, 32):
        assert ch(3, co) == B.Kernel.TILED, co
    for co in (48, 64):
        assert ch(3, co) == B.Kernel.SCALAR and ch(3, co, 1, 2) == B.Kernel.SCALAR, co
        assert ch(3, co, 3) == B.Kernel.TILED and ch(3, co, 7, 2) == B.Kernel.TILED, co
    for co in (128, 256):
        assert ch(3, co, 3) == B.Kernel.SCALAR, co


def test_mi355x_dispatch_table():
    for name, wl in WORKLOADS.items():
        dt = B.Dtype.F16 if wl.dtype == "f16" else B.Dtype.F32
        got = B.dispatch_choose(wl.N, wl.H, wl.W, wl.C_in, wl.C_out, wl.kh, wl.kw, wl.stride,
                                wl.pad, dt, B.Table.MI355X)
        if wl.dtype == "f32":
            assert got == B.Kernel.SCALAR
        elif wl.C_in % 8 == 0:
            assert got == B.Kernel.IGEMM, name
        else:
            assert got in (B.Kernel.TILED, B.Kernel.IGEMM, B.Kernel.SCALAR), name


def test_run_argument_errors_before_any_launch(lib):
    st, h = _create(lib, 2, 16, 16, 16, 32, 3, 3, 1, 1, kernel=3)
    assert st == OK
    a = 1 << 20  # aligned fake addresses: never dereferenced on these paths
    run = lib.tg_conv_bn_silu_run
    assert run(None, a, a, a, a, a, None, 0, None) == INVAL
    assert run(h, None, a, a, a, a, None, 0, None) == INVAL
    assert run(h, a, a, a, a, None, None, 0, None) == INVAL
    assert run(h, a + 2, a, a, a, a, None, 0, None) == ALIGN
    assert run(h, a, a + 4, a, a, a, None, 0, None) == ALIGN
    assert run(h, a, a, a, a, a + 8, None, 0, None) == ALIGN
    lib.tg_conv_bn_silu_destroy(h)
    st, h = _create(lib, 2, 16, 16, 16, 32, 3, 3, 1, 1, kernel=0x100)
    assert st == OK
    assert run(h, a, a, a, a, a, None, 0, None) == WS
    assert run(h, a, a, a, a, a, a, 10, None) == WS
    lib.tg_conv_bn_silu_destroy(h)


def test_packed_filter_host_logic(lib):
    """Packed-filter sizes (nk chunks x ceil(C_out/16) blocks x 2 KB) for the
    patch-staged plans, and every error that returns before a launch."""
    sz = ctypes.c_size_t()
    q = lib.tg_conv_bn_silu_packed_filter_bytes
    for shape, kernel, want in [
            ((32, 28, 28, 128, 128, 3, 3, 1, 1), 0, 18 * 8 * 2048),   # the 3x3 layer
            ((16, 56, 56, 64, 64, 7, 7, 1, 3), 0, 49 * 4 * 2048),     # the 7x7 layer
            ((2, 12, 12, 64, 33, 3, 3, 1, 1), 3, 9 * 3 * 2048)]:      # partial block
        st, h = _create(lib, *shape, kernel=kernel)
        assert st == OK
        buf = ctypes.create_string_buffer(256)
        lib.tg_conv_bn_silu_describe(h, buf, 256)
        assert b"igemm_patch" in buf.value, buf.value
        assert q(h, ctypes.byref(sz)) == OK and sz.value == want
        assert q(h, None) == INVAL
        a = 1 << 20
        pack = lib.tg_conv_bn_silu_pack_filter
        assert pack(None, a, 2 * a, want, None) == INVAL
        assert pack(h, a, a, want, None) == INVAL
        assert pack(h, a, 2 * a, want - 16, None) == WS
        assert pack(h, a + 8, 2 * a, want, None) == ALIGN
        runp = lib.tg_conv_bn_silu_run_packed
        assert runp(h, None, a, a, a, a, None) == INVAL
        assert runp(h, a + 2, a, a, a, a, None) == ALIGN
        assert runp(h, a, a + 8, a, a, a, None) == ALIGN
        lib.tg_conv_bn_silu_destroy(h)
    assert q(None, ctypes.byref(sz)) == INVAL
    for shape, kernel in [((32, 56, 56, 64, 256, 1, 1, 1, 0), 0),    # 1x1 kernel
                          ((32, 28, 28, 128, 128, 3, 3, 1, 1), 0x100),  # unfused
                          ((2, 16, 16, 16, 32, 3, 3, 1, 1), 0)]:     # C_in % 64 != 0
        st, h = _create(lib, *shape, kernel=kernel)
        assert st == OK
        sz.value = 7
        assert q(h, ctypes.byref(sz)) == UNSUP and sz.value == 0
        a = 1 << 20
        assert lib.tg_conv_bn_silu_pack_filter(h, a, 2 * a, 1 << 30, None) == UNSUP
        assert lib.tg_conv_bn_silu_run_packed(h, a, a, a, a, a, None) == UNSUP
        lib.tg_conv_bn_silu_destroy(h)


def test_train_argument_errors_before_any_launch(lib):
    """Training-mode entry: argument checks return before any launch."""
    st, h = _create(lib, 2, 16, 16, 16, 32, 3, 3, 1, 1)
    assert st == OK
    ws = ctypes.c_size_t()
    assert lib.tg_conv_bn_silu_train_workspace(h, ctypes.byref(ws)) == OK
    # t1 lives in y: the workspace holds scale and bias (256 bytes each,
    # rounded) and the fp64 (sum, sum of squares) of 8 row blocks of 64 rows
    # (M = 512) for 32 channels.
    assert ws.value == 2 * 256 + 8 * 32 * 2 * 8
    assert lib.tg_conv_bn_silu_train_workspace(None, ctypes.byref(ws)) == INVAL
    a = 1 << 20  # aligned fake addresses: never dereferenced on these paths
    tr = lib.tg_conv_bn_silu_train_run
    n = ws.value
    assert tr(None, a, a, a, a, 1e-5, 0.1, a, a, a, a, a, a, n, None) == INVAL
    assert tr(h, a, a, None, a, 1e-5, 0.1, a, a, a, a, a, a, n, None) == INVAL
    assert tr(h, a, a, a, a, 1e-5, 0.1, a, None, a, a, a, a, n, None) == INVAL   # one running
    assert tr(h, a, a, a, a, -1.0, 0.1, a, a, a, a, a, a, n, None) == INVAL
    assert tr(h, a, a, a, a, 1e-5, 1.5, a, a, a, a, a, a, n, None) == INVAL
    assert tr(h, a, a, a, a, 1e-5, 0.1, a, a, a, a, a, None, n, None) == WS
    assert tr(h, a, a, a, a, 1e-5, 0.1, a, a, a, a, a, a, n - 1, None) == WS
    lib.tg_conv_bn_silu_destroy(h)
    st, h = _create(lib, 1, 1, 1, 8, 16, 1, 1, 1, 0)  # one output pixel: M = 1
    assert st == OK
    assert lib.tg_conv_bn_silu_train_workspace(h, ctypes.byref(ws)) == OK
    assert tr(h, a, a, a, a, 1e-5, 0.1, None, None, a, a, a, a, ws.value, None) == INVAL
    lib.tg_conv_bn_silu_destroy(h)


def test_layout_argument_errors(lib):
    a, b = 1 << 20, 1 << 21  # fake addresses: never dereferenced on these paths
    for fn in (lib.tg_nchw_to_nhwc, lib.tg_nhwc_to_nchw, lib.tg_filter_oihw_to_ohwi):
        assert fn(None, b, 1, 2, 3, 4, 0, None) == INVAL
        assert fn(a, None, 1, 2, 3, 4, 0, None) == INVAL
        assert fn(a, a, 1, 2, 3, 4, 0, None) == INVAL
        assert fn(a, b, 0, 2, 3, 4, 0, None) == INVAL
        assert fn(a, b, 1, 2, 3, -4, 0, None) == INVAL
        assert fn(a, b, 1, 2, 3, 4, 7, None) == 2
        assert fn(a, b, 1024, 1024, 64, 64, 0, None) == 2  # 2^32 elements


def test_bn_fold_argument_errors(lib):
    a = 1 << 20
    f = lib.tg_bn_fold
    assert f(None, a, a, a, 1e-5, 4, a, a, None) == INVAL
    assert f(a, a, a, a, 1e-5, 0, a, a, None) == INVAL
    assert f(a, a, a, a, -1.0, 4, a, a, None) == INVAL
    assert f(a, a, a, a, float("nan"), 4, a, a, None) == INVAL


def test_split_workspace_size(lib):
    """Split form (conv -> t1, then one bn+silu kernel): one intermediate."""
    wl = WORKLOADS["conv3x3_c128_k128"]
    st, h = _create(lib, wl.N, wl.H, wl.W, wl.C_in, wl.C_out, 3, 3, 1, 1, kernel=0x200)
    assert st == OK
    k, ws = ctypes.c_int(), ctypes.c_size_t()
    lib.tg_conv_bn_silu_query(h, None, None, ctypes.byref(k), ctypes.byref(ws))
    ybytes = wl.N * wl.P * wl.Q * wl.C_out * 2
    assert ws.value == (ybytes + 255) // 256 * 256
    assert k.value == (3 | 0x200)
    buf = ctypes.create_string_buffer(256)
    assert lib.tg_conv_bn_silu_describe(h, buf, 256) == OK
    assert buf.value.decode().startswith("split:")
    lib.tg_conv_bn_silu_destroy(h)
    # the two baselines exclude each other
    st, h = _create(lib, wl.N, wl.H, wl.W, wl.C_in, wl.C_out, 3, 3, 1, 1, kernel=0x300)
    assert st == 2 and not h


def test_strings(lib):
    for s in range(6):
        assert B.status_string(s)
    assert B.status_string(99) == "unknown status"
    assert B.kernel_name(3) == "conv2d_bn_silu_igemm"
    assert B.kernel_name(3 | 0x100) == "unfused(igemm)"
    assert B.kernel_name(1 | 0x200) == "split(scalar)"
    assert B.kernel_name(3 | 0x300) == "unknown kernel"
    assert B.kernel_name(77) == "unknown kernel"


def _create_tuned(lib, shape, tuning, kernel=0, act=0, dtype=0, y_dtype=0):
    h = ctypes.c_void_p()
    st = lib.tg_conv_bn_silu_create_tuned(ctypes.byref(h), *shape, dtype, kernel, act, y_dtype,
                                          tuning)
    return st, h


def _describe(lib, h):
    buf = ctypes.create_string_buffer(512)
    assert lib.tg_conv_bn_silu_describe(h, buf, 512) == OK
    return buf.value.decode()


HEAD = (32, 56, 56, 64, 256, 1, 1, 1, 0)


def test_tuned_create_overrides_are_explicit(lib):
    """Kernel-variant overrides travel in the tuning string and nowhere else:
    NULL and "" give the default plan, known keys change it, and the plan
    text shows the forced variant."""
    st, h0 = _create(lib, *HEAD)
    assert st == OK
    default = _describe(lib, h0)
    for t in (None, b""):
        st, h = _create_tuned(lib, HEAD, t)
        assert st == OK and _describe(lib, h) == default
        lib.tg_conv_bn_silu_destroy(h)
    st, h = _create_tuned(lib, HEAD, b"cu=2,cu_pd=1")
    assert st == OK
    d = _describe(lib, h)
    assert "igemm_cu" in d and "waves=8" in d and "pd=1" in d, d
    lib.tg_conv_bn_silu_destroy(h)
    st, h = _create_tuned(lib, HEAD, b"cu=0")
    assert st == OK and "igemm_rw" in _describe(lib, h)
    lib.tg_conv_bn_silu_destroy(h)
    stem = (64, 224, 224, 3, 16, 3, 3, 2, 1)
    st, h = _create_tuned(lib, stem, b"stem=0,tm_pipe=0,tm_rows=4")
    assert st == OK and _describe(lib, h).startswith("tiled_mfma R=4"), _describe(lib, h)
    lib.tg_conv_bn_silu_destroy(h)
    # The band implicit GEMM is opt-in; it takes no packed filter.
    c2 = (32, 28, 28, 128, 128, 3, 3, 1, 1)
    st, h = _create(lib, *c2)
    assert st == OK and _describe(lib, h).startswith("igemm_patch"), _describe(lib, h)
    lib.tg_conv_bn_silu_destroy(h)
    st, h = _create_tuned(lib, c2, b"band=1")
    d = _describe(lib, h)
    assert st == OK and d.startswith("igemm_band tile=112px x 128ch") and "grid=224" in d, d
    sz = ctypes.c_size_t(7)
    assert lib.tg_conv_bn_silu_packed_filter_bytes(h, ctypes.byref(sz)) == UNSUP and sz.value == 0
    lib.tg_conv_bn_silu_destroy(h)
    lib.tg_conv_bn_silu_destroy(h0)


@pytest.mark.parametrize("bad", [b"bogus=1", b"cu", b"cu=", b"cu=x", b"cu=2,", b"cu=2;cu_pd=1",
                                 b"cu=-1", b"cu=99999999", b"cu=2,,cu_pd=1", b"=3", b"cu_pd=4",
                                 b"cu_pd=0", b" cu=2"])
def test_tuned_create_rejects_bad_text(lib, bad):
    st, h = _create_tuned(lib, HEAD, bad)
    assert st == INVAL and not h.value


def test_library_reads_no_environment(lib, monkeypatch):
    """The names the library once read from the environment change nothing."""
    st, h0 = _create(lib, *HEAD)
    base = _describe(lib, h0)
    for k, v in (("TG_CU", "0"), ("TG_CU_PD", "1"), ("TG_IGEMM_CFG", "0"), ("TG_PATCH_CFG", "1"),
                 ("TG_STEM", "0"), ("TG_LOG", "1")):
        monkeypatch.setenv(k, v)
    st, h = _create(lib, *HEAD)
    assert st == OK and _describe(lib, h) == base
    lib.tg_conv_bn_silu_destroy(h)
    lib.tg_conv_bn_silu_destroy(h0)


def test_static_train_entry_rejects_oversized_plan_on_host(lib):
    """tg_conv_bn_silu_train_run_static checks the plan's training workspace
    against the static array before touching the GPU: 1024 channels over 512
    row blocks need 8 MiB of partials, above TG_STATIC_SCRATCH_BYTES (4 MiB);
    argument errors come first, as for train_run."""
    st, h = _create(lib, 64, 56, 56, 64, 1024, 1, 1, 1, 0)
    assert st == OK
    ws = ctypes.c_size_t()
    assert lib.tg_conv_bn_silu_train_workspace(h, ctypes.byref(ws)) == OK
    assert ws.value > 4 << 20
    a = 1 << 20  # fake addresses: never dereferenced on these paths
    f = lib.tg_conv_bn_silu_train_run_static
    assert f(h, a, a, a, a, 1e-5, 0.1, None, None, None, None, a, None) == UNSUP
    assert f(h, a, a, None, a, 1e-5, 0.1, None, None, None, None, a, None) == INVAL
    assert f(None, a, a, a, a, 1e-5, 0.1, None, None, None, None, a, None) == INVAL
    lib.tg_conv_bn_silu_destroy(h)
