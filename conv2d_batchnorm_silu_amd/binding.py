"""ctypes binding of libtgconv.so (include/tg_conv_bn_silu.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI. PyTorch supplies device memory (tensor data
pointers) and the current HIP stream. There is no CPU fallback: if the shared
library is missing, loading fails with an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import enum
import os
import re
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
LIB_PATH = os.path.join(_HERE, "libtgconv.so")
HEADER = os.path.join(_ROOT, "include", "tg_conv_bn_silu.h")

_lock = threading.Lock()
_lib = None


class Dtype(enum.IntEnum):
    F16 = 0
    F32 = 1
    F8_E4M3 = 2  # output only


class Kernel(enum.IntEnum):
    AUTO = 0
    SCALAR = 1
    TILED = 2
    IGEMM = 3
    UNFUSED = 0x100
    SPLIT = 0x200


class Activation(enum.IntEnum):
    SILU = 0
    RELU = 1
    GELU = 2
    NONE = 3


class Table(enum.IntEnum):
    MI355X = 0
    PAGES = 1


STATUS = {0: "TG_OK", 1: "TG_ERR_INVALID_ARGUMENT", 2: "TG_ERR_UNSUPPORTED",
          3: "TG_ERR_ALIGNMENT", 4: "TG_ERR_WORKSPACE", 5: "TG_ERR_HIP"}
ERR_UNSUPPORTED = 2


class TgError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, STATUS.get(status, status),
                                                 status_string(status)))


def library_path() -> str:
    return LIB_PATH


def build_library() -> str:
    from .build import build_library as _b
    return _b()


def library():
    """Load libtgconv.so (once). Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtgconv.so is not built: run `python -m "
                               "conv2d_batchnorm_silu_amd.build` (or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        i, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        pp = ctypes.POINTER(ctypes.c_void_p)
        lib.tg_conv_bn_silu_create.argtypes = [pp] + [i] * 9 + [i, i]
        lib.tg_conv_bn_silu_create.restype = i
        lib.tg_conv_bn_silu_create_with_table.argtypes = [pp] + [i] * 9 + [i, i, i]
        lib.tg_conv_bn_silu_create_with_table.restype = i
        lib.tg_conv_bn_act_create.argtypes = [pp] + [i] * 9 + [i, i, i]
        lib.tg_conv_bn_act_create.restype = i
        lib.tg_conv_bn_act_create_out.argtypes = [pp] + [i] * 9 + [i, i, i, i]
        lib.tg_conv_bn_act_create_out.restype = i
        lib.tg_conv_bn_silu_create_tuned.argtypes = [pp] + [i] * 9 + [i, i, i, i, ctypes.c_char_p]
        lib.tg_conv_bn_silu_create_tuned.restype = i
        lib.tg_conv_bn_silu_run.argtypes = [vp] * 6 + [vp, sz, vp]
        lib.tg_conv_bn_silu_run.restype = i
        lib.tg_conv_bn_silu_run_residual.argtypes = [vp] * 7 + [vp]
        lib.tg_conv_bn_silu_run_residual.restype = i
        lib.tg_conv_bn_silu_packed_filter_bytes.argtypes = [vp, ctypes.POINTER(sz)]
        lib.tg_conv_bn_silu_packed_filter_bytes.restype = i
        lib.tg_conv_bn_silu_pack_filter.argtypes = [vp, vp, vp, sz, vp]
        lib.tg_conv_bn_silu_pack_filter.restype = i
        lib.tg_conv_bn_silu_run_packed.argtypes = [vp] * 6 + [vp]
        lib.tg_conv_bn_silu_run_packed.restype = i
        lib.tg_conv_bn_silu_destroy.argtypes = [vp]
        lib.tg_conv_bn_silu_destroy.restype = i
        lib.tg_bn_fold.argtypes = [vp] * 4 + [ctypes.c_float, i, vp, vp, vp]
        lib.tg_bn_fold.restype = i
        ip = ctypes.POINTER(ctypes.c_int)
        lib.tg_conv_bn_silu_query.argtypes = [vp, ip, ip, ip, ctypes.POINTER(sz)]
        lib.tg_conv_bn_silu_query.restype = i
        lib.tg_conv_bn_silu_describe.argtypes = [vp, ctypes.c_char_p, sz]
        lib.tg_conv_bn_silu_describe.restype = i
        lib.tg_dispatch_choose.argtypes = [i] * 9 + [i, i, ip]
        lib.tg_dispatch_choose.restype = i
        lib.tg_status_string.argtypes = [i]
        lib.tg_status_string.restype = ctypes.c_char_p
        lib.tg_kernel_name.argtypes = [i]
        lib.tg_kernel_name.restype = ctypes.c_char_p
        f = ctypes.c_float
        lib.tg_conv_bn_silu_train_run.argtypes = [vp] * 5 + [f, f] + [vp] * 5 + [vp, sz, vp]
        lib.tg_conv_bn_silu_train_run.restype = i
        lib.tg_conv_bn_silu_train_run_static.argtypes = [vp] * 5 + [f, f] + [vp] * 6
        lib.tg_conv_bn_silu_train_run_static.restype = i
        lib.tg_conv_bn_silu_train_workspace.argtypes = [vp, ctypes.POINTER(sz)]
        lib.tg_conv_bn_silu_train_workspace.restype = i
        for name in ("tg_filter_oihw_to_ohwi", "tg_nchw_to_nhwc", "tg_nhwc_to_nchw"):
            getattr(lib, name).argtypes = [vp, vp, i, i, i, i, i, vp]
            getattr(lib, name).restype = i
        _lib = lib
        return lib


def exported_symbols() -> list:
    """Function names the public header declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_[a-z0-9_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return library().tg_status_string(int(status)).decode()


def kernel_name(k: int) -> str:
    return library().tg_kernel_name(int(k)).decode()


def _check(st: int, where: str):
    if st != 0:
        raise TgError(st, where)


def dispatch_choose(N, H, W, C_in, C_out, kh, kw, stride, pad, dtype=Dtype.F16,
                    table=Table.MI355X) -> Kernel:
    out = ctypes.c_int(-1)
    _check(library().tg_dispatch_choose(N, H, W, C_in, C_out, kh, kw, stride, pad, int(dtype),
                                        int(table), ctypes.byref(out)), "tg_dispatch_choose")
    return Kernel(out.value)


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_TORCH_DTYPE = {}


def _torch_dtype(dt: Dtype):
    import torch
    return {Dtype.F16: torch.float16, Dtype.F32: torch.float32,
            Dtype.F8_E4M3: torch.float8_e4m3fn}[Dtype(dt)]


def _as_dtype(d) -> Dtype:
    if isinstance(d, Dtype):
        return d
    return {"f16": Dtype.F16, "fp16": Dtype.F16, "float16": Dtype.F16,
            "f32": Dtype.F32, "fp32": Dtype.F32, "float32": Dtype.F32,
            "f8": Dtype.F8_E4M3, "fp8": Dtype.F8_E4M3, "f8_e4m3": Dtype.F8_E4M3}[str(d)]


def tuning_string(tuning) -> bytes | None:
    """A dict {key: int} (or a ready "key=value,..." string) as the tuning
    text tg_conv_bn_silu_create_tuned takes; None for no overrides."""
    if tuning is None:
        return None
    if isinstance(tuning, (str, bytes)):
        return tuning.encode() if isinstance(tuning, str) else tuning
    return ",".join("%s=%d" % (k, int(v)) for k, v in sorted(tuning.items())).encode()


def _as_kernel(k) -> int:
    if isinstance(k, (int, Kernel)):
        return int(k)
    names = {"auto": 0, "scalar": 1, "tiled": 2, "igemm": 3}
    s = str(k)
    for prefix, flag in (("unfused", Kernel.UNFUSED), ("split", Kernel.SPLIT)):
        if s.startswith(prefix):
            inner = s[len(prefix):].strip("_:()") or "auto"
            return names[inner] | flag
    return names[s]


class ConvBnSilu:
    """One planned fused conv2d + BatchNorm + SiLU shape.

    ``run(x, w, scale, bias)`` takes device tensors: x NHWC [N,H,W,C_in], w
    OHWI [C_out,kh,kw,C_in] in the plan's dtype, scale/bias fp32 [C_out]
    (from ``bn_fold``); it returns y NHWC [N,P,Q,C_out] (or writes ``out``).
    ``tuning`` ({key: int} or "key=value,...") selects kernel variants
    explicitly (tg_conv_bn_silu_create_tuned); the library reads no
    environment variables.
    """

    def __init__(self, N, H, W, C_in, C_out, kh, kw=None, stride=1, pad=0, dtype="f16",
                 kernel="auto", table=Table.MI355X, act="silu", out_dtype=None, tuning=None):
        kw = kh if kw is None else kw
        self.shape = (N, H, W, C_in, C_out, kh, kw, stride, pad)
        self.dtype = _as_dtype(dtype)
        self.out_dtype = self.dtype if out_dtype is None else _as_dtype(out_dtype)
        self.act = Activation[str(act).upper()] if not isinstance(act, Activation) else act
        self._lib = library()
        h = ctypes.c_void_p()
        self.tuning = tuning_string(tuning)
        if self.tuning is not None:
            if table != Table.MI355X:
                raise ValueError("tuning overrides use the MI355X dispatch table")
            st = self._lib.tg_conv_bn_silu_create_tuned(
                ctypes.byref(h), N, H, W, C_in, C_out, kh, kw, stride, pad, int(self.dtype),
                _as_kernel(kernel), int(self.act), int(self.out_dtype), self.tuning)
        elif self.out_dtype != self.dtype:
            if table != Table.MI355X:
                raise ValueError("an fp8 output uses the MI355X dispatch table")
            st = self._lib.tg_conv_bn_act_create_out(
                ctypes.byref(h), N, H, W, C_in, C_out, kh, kw, stride, pad, int(self.dtype),
                _as_kernel(kernel), int(self.act), int(self.out_dtype))
        elif self.act == Activation.SILU:
            st = self._lib.tg_conv_bn_silu_create_with_table(
                ctypes.byref(h), N, H, W, C_in, C_out, kh, kw, stride, pad, int(self.dtype),
                _as_kernel(kernel), int(table))
        else:
            if table != Table.MI355X:
                raise ValueError("activations other than SiLU use the MI355X dispatch table")
            st = self._lib.tg_conv_bn_act_create(
                ctypes.byref(h), N, H, W, C_in, C_out, kh, kw, stride, pad, int(self.dtype),
                _as_kernel(kernel), int(self.act))
        _check(st, "tg_conv_bn_silu_create")
        self._h = h
        P, Q, ch, ws = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_size_t()
        _check(self._lib.tg_conv_bn_silu_query(h, ctypes.byref(P), ctypes.byref(Q),
                                               ctypes.byref(ch), ctypes.byref(ws)),
               "tg_conv_bn_silu_query")
        self.P, self.Q = P.value, Q.value
        self.kernel = ch.value
        self.workspace_bytes = ws.value
        self._ws = None

    @property
    def y_shape(self):
        N, C_out = self.shape[0], self.shape[4]
        return (N, self.P, self.Q, C_out)

    def describe(self) -> str:
        buf = ctypes.create_string_buffer(512)
        _check(self._lib.tg_conv_bn_silu_describe(self._h, buf, 512), "tg_conv_bn_silu_describe")
        return buf.value.decode()

    def kernel_name(self) -> str:
        return kernel_name(self.kernel)

    def _check_tensor(self, t, shape, dtype, name):
        if not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)
        if t.dtype != dtype:
            raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)

    def run_ptr(self, x, w, scale, bias, y, workspace=0, workspace_bytes=0, stream=None) -> int:
        """Raw call with integer device addresses; returns the tg_status."""
        return self._lib.tg_conv_bn_silu_run(self._h, x, w, scale, bias, y, workspace,
                                             workspace_bytes, _stream_handle(stream))

    def run(self, x, w, scale, bias, out=None, workspace=None, stream=None, residual=None):
        """y = act(BN(conv(x, w))) (+ residual, a tensor of y's shape and dtype)."""
        import torch
        N, H, W, C_in, C_out, kh, kw, stride, pad = self.shape
        td = _torch_dtype(self.dtype)
        self._check_tensor(x, (N, H, W, C_in), td, "x")
        self._check_tensor(w, (C_out, kh, kw, C_in), td, "w")
        self._check_tensor(scale, (C_out,), torch.float32, "scale")
        self._check_tensor(bias, (C_out,), torch.float32, "bias")
        yd = _torch_dtype(self.out_dtype)
        if out is None:
            out = torch.empty(self.y_shape, dtype=yd, device=x.device)
        self._check_tensor(out, self.y_shape, yd, "out")
        ws_ptr, ws_bytes = 0, 0
        if self.workspace_bytes:
            if workspace is None:
                if self._ws is None or self._ws.device != x.device:
                    self._ws = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=x.device)
                workspace = self._ws
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        if residual is not None:
            self._check_tensor(residual, self.y_shape, yd, "residual")
            st = self._lib.tg_conv_bn_silu_run_residual(
                self._h, x.data_ptr(), w.data_ptr(), scale.data_ptr(), bias.data_ptr(),
                residual.data_ptr(), out.data_ptr(), _stream_handle(stream))
            _check(st, "tg_conv_bn_silu_run_residual")
            return out
        st = self.run_ptr(x.data_ptr(), w.data_ptr(), scale.data_ptr(), bias.data_ptr(),
                          out.data_ptr(), ws_ptr, ws_bytes, stream)
        _check(st, "tg_conv_bn_silu_run")
        return out

    __call__ = run

    def packed_filter_bytes(self) -> int:
        """Bytes of this plan's load-time packed filter; 0 if its kernel takes
        only the OHWI filter."""
        n = ctypes.c_size_t()
        st = self._lib.tg_conv_bn_silu_packed_filter_bytes(self._h, ctypes.byref(n))
        if st == ERR_UNSUPPORTED:
            return 0
        _check(st, "tg_conv_bn_silu_packed_filter_bytes")
        return n.value

    def pack_filter(self, w, out=None, stream=None):
        """The OHWI filter w re-packed once into this plan's kernel tile order
        (a uint8 device tensor of packed_filter_bytes())."""
        import torch
        N, H, W, C_in, C_out, kh, kw, stride, pad = self.shape
        self._check_tensor(w, (C_out, kh, kw, C_in), _torch_dtype(self.dtype), "w")
        n = self.packed_filter_bytes()
        if n == 0:
            raise TgError(ERR_UNSUPPORTED, "tg_conv_bn_silu_packed_filter_bytes")
        if out is None:
            out = torch.empty(n, dtype=torch.uint8, device=w.device)
        self._check_tensor(out, (n,), torch.uint8, "out")
        _check(self._lib.tg_conv_bn_silu_pack_filter(self._h, w.data_ptr(), out.data_ptr(), n,
                                                     _stream_handle(stream)),
               "tg_conv_bn_silu_pack_filter")
        return out

    def run_packed(self, x, w_packed, scale, bias, out=None, stream=None):
        """run() with a filter from pack_filter(); bit-identical output."""
        import torch
        N, H, W, C_in, C_out, kh, kw, stride, pad = self.shape
        self._check_tensor(x, (N, H, W, C_in), _torch_dtype(self.dtype), "x")
        self._check_tensor(w_packed, (self.packed_filter_bytes(),), torch.uint8, "w_packed")
        self._check_tensor(scale, (C_out,), torch.float32, "scale")
        self._check_tensor(bias, (C_out,), torch.float32, "bias")
        yd = _torch_dtype(self.out_dtype)
        if out is None:
            out = torch.empty(self.y_shape, dtype=yd, device=x.device)
        self._check_tensor(out, self.y_shape, yd, "out")
        _check(self._lib.tg_conv_bn_silu_run_packed(self._h, x.data_ptr(), w_packed.data_ptr(),
                                                    scale.data_ptr(), bias.data_ptr(),
                                                    out.data_ptr(), _stream_handle(stream)),
               "tg_conv_bn_silu_run_packed")
        return out

    def train_workspace_bytes(self) -> int:
        ws = ctypes.c_size_t()
        _check(self._lib.tg_conv_bn_silu_train_workspace(self._h, ctypes.byref(ws)),
               "tg_conv_bn_silu_train_workspace")
        return ws.value

    def run_train(self, x, w, gamma, beta, eps=1e-5, momentum=0.1, running_mean=None,
                  running_var=None, out=None, workspace=None, stream=None):
        """Training-mode BatchNorm (batch statistics): returns (y, batch_mean,
        batch_var); running_mean/running_var (fp32 [C_out]) are updated in
        place when given."""
        import torch
        N, H, W, C_in, C_out, kh, kw, _, _ = self.shape
        td = _torch_dtype(self.dtype)
        self._check_tensor(x, (N, H, W, C_in), td, "x")
        self._check_tensor(w, (C_out, kh, kw, C_in), td, "w")
        for t, name in ((gamma, "gamma"), (beta, "beta")):
            self._check_tensor(t, (C_out,), torch.float32, name)
        if (running_mean is None) != (running_var is None):
            raise ValueError("give both running_mean and running_var, or neither")
        for t, name in ((running_mean, "running_mean"), (running_var, "running_var")):
            if t is not None:
                self._check_tensor(t, (C_out,), torch.float32, name)
        if out is None:
            out = torch.empty(self.y_shape, dtype=td, device=x.device)
        self._check_tensor(out, self.y_shape, td, "out")
        bm = torch.empty(C_out, dtype=torch.float32, device=x.device)
        bv = torch.empty(C_out, dtype=torch.float32, device=x.device)
        need = self.train_workspace_bytes()
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        ptr = lambda t: 0 if t is None else t.data_ptr()
        st = self._lib.tg_conv_bn_silu_train_run(
            self._h, x.data_ptr(), w.data_ptr(), gamma.data_ptr(), beta.data_ptr(), float(eps),
            float(momentum), ptr(running_mean), ptr(running_var), bm.data_ptr(), bv.data_ptr(),
            out.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream_handle(stream))
        _check(st, "tg_conv_bn_silu_train_run")
        return out, bm, bv

    def run_train_static(self, x, w, gamma, beta, eps=1e-5, momentum=0.1, running_mean=None,
                         running_var=None, out=None, batch_mean=None, batch_var=None,
                         stream=None):
        """run_train through tg_conv_bn_silu_train_run_static: the library's
        static device array serves as workspace, so with out, batch_mean and
        batch_var given nothing is allocated on this path."""
        import torch
        N, H, W, C_in, C_out, kh, kw, _, _ = self.shape
        td = _torch_dtype(self.dtype)
        self._check_tensor(x, (N, H, W, C_in), td, "x")
        self._check_tensor(w, (C_out, kh, kw, C_in), td, "w")
        for t, name in ((gamma, "gamma"), (beta, "beta")):
            self._check_tensor(t, (C_out,), torch.float32, name)
        if (running_mean is None) != (running_var is None):
            raise ValueError("give both running_mean and running_var, or neither")
        for t, name in ((running_mean, "running_mean"), (running_var, "running_var")):
            if t is not None:
                self._check_tensor(t, (C_out,), torch.float32, name)
        if out is None:
            out = torch.empty(self.y_shape, dtype=td, device=x.device)
        self._check_tensor(out, self.y_shape, td, "out")
        if batch_mean is None:
            batch_mean = torch.empty(C_out, dtype=torch.float32, device=x.device)
        if batch_var is None:
            batch_var = torch.empty(C_out, dtype=torch.float32, device=x.device)
        self._check_tensor(batch_mean, (C_out,), torch.float32, "batch_mean")
        self._check_tensor(batch_var, (C_out,), torch.float32, "batch_var")
        ptr = lambda t: 0 if t is None else t.data_ptr()
        st = self._lib.tg_conv_bn_silu_train_run_static(
            self._h, x.data_ptr(), w.data_ptr(), gamma.data_ptr(), beta.data_ptr(), float(eps),
            float(momentum), ptr(running_mean), ptr(running_var), batch_mean.data_ptr(),
            batch_var.data_ptr(), out.data_ptr(), _stream_handle(stream))
        _check(st, "tg_conv_bn_silu_train_run_static")
        return out, batch_mean, batch_var

    def close(self):
        if getattr(self, "_h", None):
            self._lib.tg_conv_bn_silu_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _layout(name, src, dst_shape, dims, stream):
    import torch
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    dt = {torch.float16: Dtype.F16, torch.float32: Dtype.F32}[src.dtype]
    dst = torch.empty(dst_shape, dtype=src.dtype, device=src.device)
    _check(getattr(library(), name)(src.data_ptr(), dst.data_ptr(), *dims, int(dt),
                                    _stream_handle(stream)), name)
    return dst


def filter_oihw_to_ohwi(w, stream=None):
    """[C_out, C_in, kh, kw] (PyTorch) -> [C_out, kh, kw, C_in], on the device."""
    O, I, kh, kw = w.shape
    return _layout("tg_filter_oihw_to_ohwi", w, (O, kh, kw, I), (O, I, kh, kw), stream)


def nchw_to_nhwc(x, stream=None):
    N, C, H, W = x.shape
    return _layout("tg_nchw_to_nhwc", x, (N, H, W, C), (N, C, H, W), stream)


def nhwc_to_nchw(y, stream=None):
    N, H, W, C = y.shape
    return _layout("tg_nhwc_to_nchw", y, (N, C, H, W), (N, C, H, W), stream)


def bn_fold(gamma, beta, mean, var, eps, scale=None, bias=None, stream=None):
    """Device BatchNorm fold: returns (scale, bias) fp32 device tensors."""
    import torch
    C = gamma.numel()
    for name, t in (("gamma", gamma), ("beta", beta), ("mean", mean), ("var", var)):
        if not t.is_cuda or t.dtype != torch.float32 or t.numel() != C or not t.is_contiguous():
            raise ValueError("%s must be a contiguous fp32 device tensor of %d elements" % (name, C))
    if scale is None:
        scale = torch.empty(C, dtype=torch.float32, device=gamma.device)
    if bias is None:
        bias = torch.empty(C, dtype=torch.float32, device=gamma.device)
    st = library().tg_bn_fold(gamma.data_ptr(), beta.data_ptr(), mean.data_ptr(), var.data_ptr(),
                              float(eps), C, scale.data_ptr(), bias.data_ptr(),
                              _stream_handle(stream))
    _check(st, "tg_bn_fold")
    return scale, bias
