"""Seeded synthetic inputs for the fused conv2d + BatchNorm + SiLU path.

This module holds data recipes only: shapes, distributions and seeds. It does
none of the method's arithmetic and is shared by the tests, the benchmark and
the smoke check, so the HIP path and the CPU oracle see identical values.

Recipe (for every workload):
  * generator ``numpy.random.Generator(PCG64(seed))``;
  * draw order x, w, gamma, beta, running_mean, running_var, each drawn in
    float64 and then cast: x and w to the workload's dtype (fp16 with
    round-to-nearest-even, or fp32), the four BatchNorm vectors to fp32;
  * N(0, v) names a normal with VARIANCE v (so w ~ N(0, 1/fan_in) has
    standard deviation 1/sqrt(fan_in));
  * gamma ~ U(0.5, 1.5), beta ~ N(0, 0.1), mean ~ N(0, 0.1),
    var ~ U(0.5, 2), eps = 1e-5 as fp32.
Layouts: x NHWC [N][H][W][C_in], w OHWI [C_out][kh][kw][C_in].

The shapes stand in for the vision-model layers that "Fusing an Epilogue"
(teenygrad docs), section "The problem", has in mind: a 1x1 channel-mixing
conv, a 3x3 body conv, a stride-2 RGB stem with few output channels and a
7x7 large-window conv ("When the fusion you want is impossible, fuse into the
producer", section "The second reason, which matters more").
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

EPS = np.float32(1e-5)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    N: int
    H: int
    W: int
    C_in: int
    C_out: int
    kh: int
    kw: int
    stride: int
    pad: int
    dtype: str  # "f16" or "f32": dtype of x, w and y
    x_dist: tuple = ("normal", 1.0)  # ("normal", variance) or ("uniform", lo, hi)
    w_var: float | None = None  # default 1 / (kh * kw * C_in)
    note: str = field(default="", compare=False)

    @property
    def P(self) -> int:
        return (self.H + 2 * self.pad - self.kh) // self.stride + 1

    @property
    def Q(self) -> int:
        return (self.W + 2 * self.pad - self.kw) // self.stride + 1

    @property
    def x_shape(self):
        return (self.N, self.H, self.W, self.C_in)

    @property
    def w_shape(self):
        return (self.C_out, self.kh, self.kw, self.C_in)

    @property
    def y_shape(self):
        return (self.N, self.P, self.Q, self.C_out)

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32_3x3", 0, 1, 16, 16, 3, 8, 3, 3, 1, 1, "f32", ("uniform", -1.0, 1.0),
                 note="fp32 3x3 on a 16x16 RGB image; oracle in milliseconds"),
        Workload("conv1x1_c64_k256", 1, 32, 56, 56, 64, 256, 1, 1, 1, 0, "f16",
                 note="1x1 conv as a GEMM: M=100352, K=64, N=256"),
        Workload("conv3x3_c128_k128", 2, 32, 28, 28, 128, 128, 3, 3, 1, 1, "f16",
                 note="3x3 implicit GEMM: M=25088, K=1152, N=128"),
        Workload("stem3x3s2_k16", 3, 64, 224, 224, 3, 16, 3, 3, 2, 1, "f16",
                 ("uniform", -1.0, 1.0), note="RGB stem, few output channels, 112x112 out"),
        Workload("stem3x3s2_k24", 3, 64, 224, 224, 3, 24, 3, 3, 2, 1, "f16",
                 ("uniform", -1.0, 1.0), note="RGB stem, 24 output channels, same x"),
        Workload("conv7x7_c64_k64", 4, 16, 56, 56, 64, 64, 7, 7, 1, 3, "f16",
                 note="large-window 7x7: M=50176, K=3136, N=64"),
    ]
}

# The workload the headline throughput is quoted on.
HEADLINE = "conv1x1_c64_k256"


def _np_dtype(dtype: str):
    if dtype == "f16":
        return np.float16
    if dtype == "f32":
        return np.float32
    raise ValueError("dtype must be 'f16' or 'f32'")


def _draw_x(rng, shape, dist):
    if dist[0] == "normal":
        return rng.normal(0.0, np.sqrt(dist[1]), size=shape)
    if dist[0] == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape)
    raise ValueError("unknown distribution %r" % (dist,))


def make_inputs(wl: Workload, seed: int | None = None) -> dict:
    """Draw x, w and the four BatchNorm vectors for ``wl`` (see module doc)."""
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    dt = _np_dtype(wl.dtype)
    x = _draw_x(rng, wl.x_shape, wl.x_dist).astype(dt)
    w_var = wl.w_var if wl.w_var is not None else 1.0 / (wl.kh * wl.kw * wl.C_in)
    w = rng.normal(0.0, np.sqrt(w_var), size=wl.w_shape).astype(dt)
    C = wl.C_out
    gamma = rng.uniform(0.5, 1.5, size=C).astype(np.float32)
    beta = rng.normal(0.0, np.sqrt(0.1), size=C).astype(np.float32)
    mean = rng.normal(0.0, np.sqrt(0.1), size=C).astype(np.float32)
    var = rng.uniform(0.5, 2.0, size=C).astype(np.float32)
    return dict(x=x, w=w, gamma=gamma, beta=beta, mean=mean, var=var, eps=EPS)


def random_small_workloads(count: int, seed: int, dtype: str = "f16", **limits) -> list:
    """Random small shapes for the parity sweep (tails, odd channel counts,
    strides up to 3, pads up to 3). Shapes only; draw data with make_inputs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    max_hw = limits.get("max_hw", 20)
    c_in_choices = limits.get("c_in", [1, 3, 4, 8, 16, 24, 40, 64])
    c_out_choices = limits.get("c_out", [1, 7, 8, 16, 17, 31, 32, 33, 48, 64, 80])
    while len(out) < count:
        k = int(rng.choice([1, 2, 3, 5, 7]))
        kw_ = k if rng.uniform() < 0.8 else int(rng.choice([1, 3, 5]))
        s = int(rng.choice([1, 1, 2, 3]))
        p = int(rng.integers(0, min(3, k) + 1))
        H = int(rng.integers(1, max_hw + 1))
        W = int(rng.integers(1, max_hw + 1))
        if H + 2 * p < k or W + 2 * p < kw_:
            continue
        wl = Workload("rand%d" % len(out), int(rng.integers(0, 2**31 - 1)),
                      int(rng.integers(1, 4)), H, W, int(rng.choice(c_in_choices)),
                      int(rng.choice(c_out_choices)), k, kw_, s, p, dtype)
        out.append(wl)
    return out
