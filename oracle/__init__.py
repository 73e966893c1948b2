"""fp64 CPU oracle for conv2d -> BatchNorm -> SiLU.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does. It
shares no code with the HIP library (``conv2d_batchnorm_silu_amd``) and does
not import it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, no contraction); this
module builds it with gcc and wraps it with ctypes. Every function takes the
exact values the GPU path reads (fp16 or fp32 arrays) and widens them to fp64,
which is exact.

What each function follows:
  * ``conv2d`` -- the convolution of "Fusing an Epilogue" (teenygrad docs),
    section "The problem": cross-correlation, symmetric zero padding,
    NHWC x, OHWI w, NHWC output.
  * ``batchnorm`` -- same section: batch norm as a per-channel multiply and
    add, written in its unfolded inference form
    gamma * (t - mean) / sqrt(var + eps) + beta.
  * ``silu`` -- same section: v * sigmoid(v) with the logistic sigmoid.
  * ``conv_bn_silu`` / ``conv_bn_silu_at`` -- same page, section "The shape
    of it": the three applied in order to every output element.
  * ``relu``, ``gelu``, ``conv_bn_act`` -- the other activations "Fusing an
    Epilogue" (section "What an epilogue is") counts as epilogue work:
    max(v, 0) and the exact GELU v * Phi(v) = v/2 * (1 + erf(v / sqrt 2))
    (Phi the standard normal CDF), or none, after the same batch norm.
  * ``conv_bn_act_residual`` -- a residual add after the activation, the
    last of the elementwise steps "Kernel Fusion" (cheatsheet page) lists as
    fusing freely: act(batchnorm(conv2d(x, w))) + r.
  * ``round_fp8_e4m3`` -- a cast to a narrower dtype, the other epilogue
    work of that section: OCP FP8 E4M3 (3 mantissa bits, exponent bias 7,
    subnormal spacing 2^-9, largest finite 448), round to nearest even.
  * ``conv_bn_silu_train`` -- batch norm with batch statistics (training
    mode), the reduction case that "Kernel Fusion" (cheatsheet page, the
    passages on reductions and on synchronization boundaries) sets apart:
    per output channel, the mean and the biased variance over all N*P*Q
    conv outputs normalise the batch (the batch-normalising transform of
    Ioffe and Szegedy, 2015); running estimates, if given, move by
    ``momentum`` towards the batch mean and the unbiased batch variance.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_llp = ctypes.POINTER(ctypes.c_longlong)


_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c99",
           "-Wall", "-Werror"]


def _compile(src: str, out: str, extra=()):
    cmd = ["gcc"] + _CFLAGS + list(extra) + ["-o", out, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (no fast-math, no
    floating-point contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    _compile(_SRC, tmp)
    os.replace(tmp, _LIB)
    return _LIB


def source() -> str:
    """The text of oracle.c (for the tests that build altered copies)."""
    with open(_SRC) as f:
        return f.read()


def _configure(lib):
    i = ctypes.c_int
    lib.oracle_out_extent.restype = ctypes.c_longlong
    lib.oracle_out_extent.argtypes = [ctypes.c_longlong] * 4
    lib.oracle_conv2d.restype = i
    lib.oracle_conv2d.argtypes = [_dp, _dp] + [i] * 9 + [_dp, i]
    lib.oracle_batchnorm.restype = None
    lib.oracle_batchnorm.argtypes = [_dp, ctypes.c_longlong, i, _dp, _dp, _dp, _dp,
                                     ctypes.c_double, _dp]
    lib.oracle_silu.restype = None
    lib.oracle_silu.argtypes = [_dp, ctypes.c_longlong, _dp]
    lib.oracle_conv_bn_silu.restype = i
    lib.oracle_conv_bn_silu.argtypes = ([_dp, _dp] + [i] * 9 + [_dp] * 4
                                        + [ctypes.c_double, _dp, i])
    lib.oracle_conv_bn_silu_at.restype = i
    lib.oracle_conv_bn_silu_at.argtypes = ([_dp, _dp] + [i] * 9 + [_dp] * 4
                                           + [ctypes.c_double, _llp, ctypes.c_longlong, _dp])
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


@contextlib.contextmanager
def altered(text: str, workdir: str):
    """Test hook: build ``text`` (an altered copy of oracle.c) in ``workdir``
    and route every function of this module through it inside the block --
    how the tests check that a planted mistake in the oracle fails a pin."""
    global _lib
    src = os.path.join(workdir, "oracle_altered.c")
    so = os.path.join(workdir, "liboracle_altered_%d.so" % abs(hash(text)))
    with open(src, "w") as f:
        f.write(text)
    _compile(src, so)
    alt = _configure(ctypes.CDLL(so))
    prev = _load()
    with _lock:
        _lib = alt
    try:
        yield
    finally:
        with _lock:
            _lib = prev


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def default_threads() -> int:
    """Host threads for the oracle: OMP_NUM_THREADS when set (a machine's
    share of its cores), else every core up to 64."""
    try:
        n = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        n = 0
    return max(1, min(n if n > 0 else (os.cpu_count() or 1), 64))


def out_extent(n_in: int, k: int, stride: int, pad: int) -> int:
    """floor((n_in + 2 pad - k) / stride) + 1, or 0 when the window does not fit."""
    return int(_load().oracle_out_extent(n_in, k, stride, pad))


def _geom(x, w, stride, pad):
    N, H, W, C_in = x.shape
    C_out, kh, kw, C_in_w = w.shape
    if C_in_w != C_in:
        raise ValueError("C_in of x and w differ")
    P, Q = out_extent(H, kh, stride, pad), out_extent(W, kw, stride, pad)
    if P == 0 or Q == 0:
        raise ValueError("window larger than the padded input")
    return N, H, W, C_in, C_out, kh, kw, P, Q


def conv2d(x, w, stride: int, pad: int, threads: int | None = None) -> np.ndarray:
    """Convolution alone. x [N,H,W,C_in], w [C_out,kh,kw,C_in] -> [N,P,Q,C_out] fp64."""
    x, w = _f64(x), _f64(w)
    N, H, W, C_in, C_out, kh, kw, P, Q = _geom(x, w, stride, pad)
    out = np.empty((N, P, Q, C_out), np.float64)
    rc = _load().oracle_conv2d(_ptr(x), _ptr(w), N, H, W, C_in, C_out, kh, kw, stride, pad,
                               _ptr(out), threads or default_threads())
    if rc:
        raise ValueError("oracle_conv2d rejected the arguments (%d)" % rc)
    return out


def batchnorm(t, gamma, beta, mean, var, eps: float) -> np.ndarray:
    """Inference batch norm over the last (channel) axis, unfolded form."""
    t = _f64(t)
    C = t.shape[-1]
    g, b, m, v = (_f64(a).reshape(C) for a in (gamma, beta, mean, var))
    out = np.empty_like(t)
    _load().oracle_batchnorm(_ptr(t), t.size // C, C, _ptr(g), _ptr(b), _ptr(m), _ptr(v),
                             float(eps), _ptr(out))
    return out


def silu(t) -> np.ndarray:
    """v * sigmoid(v), elementwise."""
    t = _f64(t)
    out = np.empty_like(t)
    _load().oracle_silu(_ptr(t), t.size, _ptr(out))
    return out


def conv_bn_silu(x, w, gamma, beta, mean, var, eps: float, stride: int, pad: int,
                 threads: int | None = None) -> np.ndarray:
    """The whole path: silu(batchnorm(conv2d(x, w))), fp64 [N,P,Q,C_out]."""
    x, w = _f64(x), _f64(w)
    N, H, W, C_in, C_out, kh, kw, P, Q = _geom(x, w, stride, pad)
    g, b, m, v = (_f64(a).reshape(C_out) for a in (gamma, beta, mean, var))
    out = np.empty((N, P, Q, C_out), np.float64)
    rc = _load().oracle_conv_bn_silu(_ptr(x), _ptr(w), N, H, W, C_in, C_out, kh, kw, stride, pad,
                                     _ptr(g), _ptr(b), _ptr(m), _ptr(v), float(eps), _ptr(out),
                                     threads or default_threads())
    if rc:
        raise ValueError("oracle_conv_bn_silu rejected the arguments (%d)" % rc)
    return out


def conv_bn_silu_at(x, w, gamma, beta, mean, var, eps: float, stride: int, pad: int,
                    flat_idx) -> np.ndarray:
    """The whole path at selected flat indices into the [N,P,Q,C_out] output."""
    x, w = _f64(x), _f64(w)
    N, H, W, C_in, C_out, kh, kw, P, Q = _geom(x, w, stride, pad)
    g, b, m, v = (_f64(a).reshape(C_out) for a in (gamma, beta, mean, var))
    idx = np.ascontiguousarray(np.asarray(flat_idx), dtype=np.int64)
    out = np.empty(idx.shape, np.float64)
    rc = _load().oracle_conv_bn_silu_at(_ptr(x), _ptr(w), N, H, W, C_in, C_out, kh, kw, stride,
                                        pad, _ptr(g), _ptr(b), _ptr(m), _ptr(v), float(eps),
                                        idx.ctypes.data_as(_llp), idx.size, _ptr(out))
    if rc:
        raise ValueError("oracle_conv_bn_silu_at rejected the arguments (%d)" % rc)
    return out


def conv_bn_silu_train(x, w, gamma, beta, eps: float, stride: int, pad: int,
                       running_mean=None, running_var=None, momentum: float = 0.1,
                       threads: int | None = None) -> dict:
    """Training-mode path: t = conv2d(x, w); per channel c, over the M =
    N*P*Q outputs, mean_c = sum(t)/M and var_c = sum((t - mean_c)^2)/M
    (two passes, fp64); y = silu(batchnorm(t, gamma, beta, mean, var, eps)).
    With running estimates: running_mean <- (1-momentum)*running_mean +
    momentum*mean and running_var <- (1-momentum)*running_var +
    momentum*var*M/(M-1). Needs M >= 2. Returns y, mean, var and the new
    running estimates (None when not given), all fp64."""
    t = conv2d(x, w, stride, pad, threads)
    C = t.shape[-1]
    flat = t.reshape(-1, C)
    M = flat.shape[0]
    if M < 2:
        raise ValueError("batch statistics need at least two values per channel")
    mean = flat.sum(axis=0) / M
    var = ((flat - mean) ** 2).sum(axis=0) / M
    y = silu(batchnorm(t, gamma, beta, mean, var, eps))
    out = {"y": y, "mean": mean, "var": var, "running_mean": None, "running_var": None}
    m = float(momentum)
    if running_mean is not None:
        out["running_mean"] = (1.0 - m) * _f64(running_mean).reshape(C) + m * mean
    if running_var is not None:
        out["running_var"] = (1.0 - m) * _f64(running_var).reshape(C) + m * var * (M / (M - 1.0))
    return out


def relu(t) -> np.ndarray:
    """max(v, 0), elementwise."""
    return np.maximum(_f64(t), 0.0)


def gelu(t) -> np.ndarray:
    """v * Phi(v) with Phi(v) = (1 + erf(v / sqrt 2)) / 2, elementwise (libm
    erf through scipy)."""
    from scipy.special import erf
    t = _f64(t)
    return 0.5 * t * (1.0 + erf(t / np.sqrt(2.0)))


ACTIVATIONS = {"silu": silu, "relu": relu, "gelu": gelu, "none": lambda t: _f64(t)}


def conv_bn_act(x, w, gamma, beta, mean, var, eps: float, stride: int, pad: int, act: str,
                threads: int | None = None) -> np.ndarray:
    """act(batchnorm(conv2d(x, w))) for act in silu, relu, gelu, none."""
    return ACTIVATIONS[act](batchnorm(conv2d(x, w, stride, pad, threads), gamma, beta, mean, var,
                                      eps))


def conv_bn_act_at(x, w, gamma, beta, mean, var, eps: float, stride: int, pad: int, act: str,
                   flat_idx) -> np.ndarray:
    """conv_bn_act at selected flat indices into the [N,P,Q,C_out] output:
    each conv value is the plain window sum over an explicitly zero-padded
    copy of x, then the unfolded batch norm and the activation."""
    x, w = _f64(x), _f64(w)
    N, H, W, C_in, C_out, kh, kw, P, Q = _geom(x, w, stride, pad)
    idx = np.asarray(flat_idx, dtype=np.int64)
    n, rem = np.divmod(idx, P * Q * C_out)
    p, rem = np.divmod(rem, Q * C_out)
    q, k = np.divmod(rem, C_out)
    xp = np.pad(x, ((0, 0), (pad, pad), (pad, pad), (0, 0)))
    conv = np.array([np.sum(xp[n[i], p[i] * stride:p[i] * stride + kh,
                               q[i] * stride:q[i] * stride + kw, :] * w[k[i]])
                     for i in range(idx.size)])
    g, b, m, v = (_f64(a).reshape(C_out)[k] for a in (gamma, beta, mean, var))
    return ACTIVATIONS[act](g * (conv - m) / np.sqrt(v + eps) + b)


def round_fp8_e4m3(t) -> np.ndarray:
    """Round to the nearest OCP FP8 E4M3 value, ties to even, as fp64: the
    spacing of the representable values at |v| is 2^(e-3) with e =
    max(floor(log2 |v|), -6) (below 2^-6 the subnormals, spacing 2^-9).
    Values beyond 448 in magnitude are outside the format and returned as
    NaN (there is no infinity in E4M3)."""
    t = _f64(t)
    a = np.abs(t)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    q = np.exp2(np.maximum(e, -6.0) - 3.0)
    r = np.round(t / q) * q  # numpy rounds halves to even
    # a value just below a power of two can round up to it: still exact.
    return np.where(np.abs(r) > 448.0, np.nan, r)


def conv_bn_act_residual(x, w, gamma, beta, mean, var, eps: float, stride: int, pad: int,
                         act: str, residual, threads: int | None = None) -> np.ndarray:
    """act(batchnorm(conv2d(x, w))) + residual (residual of the output's shape)."""
    out = conv_bn_act(x, w, gamma, beta, mean, var, eps, stride, pad, act, threads)
    r = _f64(residual)
    if r.shape != out.shape:
        raise ValueError("residual shape %s differs from the output's %s" % (r.shape, out.shape))
    return out + r
