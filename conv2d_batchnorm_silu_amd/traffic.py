"""Algorithmic work of the path: HBM bytes and FLOPs per workload.

Host-side bookkeeping only (no kernel arithmetic). The byte model follows
the pages:
  * "Fusing an Epilogue" (teenygrad docs), section "The problem": run as
    three library calls, conv -> bn -> silu makes six tensor trips to
    memory (each op reads one tensor and writes one); fused, it makes two.
  * "Kernel Fusion" (GPU cheatsheet), elementwise-chain section: a chain of
    n elementwise ops over N elements moves 2nN element-trips unfused and
    2N fused.
  * "Costs and benefits of kernel fusion", traffic section: an fp16
    intermediate of E elements costs at least 2E bytes to store plus 2E bytes
    to load back.
Bytes are algorithmic: every tensor touched exactly once per kernel that
needs it. FLOPs count the convolution's multiply-adds only (2 per MAC).
"""
from __future__ import annotations

ELEM_BYTES = {"f16": 2, "f32": 4}


def chain_trips(n_ops: int) -> tuple:
    """Tensor trips (reads + writes) of an n-op chain of same-size tensors:
    (unfused, fused)."""
    if n_ops < 1:
        raise ValueError("n_ops >= 1")
    return 2 * n_ops, 2


def intermediate_bytes(elements: int, elem_bytes: int) -> int:
    """Minimum HBM bytes one materialised intermediate costs: one store and one
    later load."""
    return 2 * elements * elem_bytes


def workload_bytes(wl) -> dict:
    """Per-tensor algorithmic bytes of one fused call on workload ``wl``."""
    e = ELEM_BYTES[wl.dtype]
    x = wl.N * wl.H * wl.W * wl.C_in * e
    w = wl.C_out * wl.kh * wl.kw * wl.C_in * e
    bn = 2 * wl.C_out * 4  # folded scale and bias, fp32
    y = wl.N * wl.P * wl.Q * wl.C_out * e
    return dict(x=x, w=w, bn=bn, y=y)


def fused_bytes(wl) -> int:
    b = workload_bytes(wl)
    return b["x"] + b["w"] + b["bn"] + b["y"]


def fused_bytes_fp8_out(wl) -> int:
    """Fused path with y stored as fp8 (one byte per element)."""
    b = workload_bytes(wl)
    return b["x"] + b["w"] + b["bn"] + b["y"] // ELEM_BYTES[wl.dtype]


def unfused_bytes(wl) -> int:
    """conv writes t1, bn reads t1 and writes t2, silu reads t2 and writes y;
    t1 and t2 have y's shape and dtype, so two intermediates are added."""
    b = workload_bytes(wl)
    return fused_bytes(wl) + 2 * intermediate_bytes(b["y"] // ELEM_BYTES[wl.dtype],
                                                   ELEM_BYTES[wl.dtype])


def split_bytes(wl) -> int:
    """conv writes t1, one bn+silu kernel reads t1 and writes y: one
    intermediate of y's shape and dtype is added."""
    b = workload_bytes(wl)
    return fused_bytes(wl) + intermediate_bytes(b["y"] // ELEM_BYTES[wl.dtype],
                                                ELEM_BYTES[wl.dtype])


def train_bytes(wl) -> int:
    """Training-mode BatchNorm as built: conv writes t1, the statistics pass
    reads t1, the BatchNorm+SiLU pass reads t1 and writes y (gamma/beta in
    place of the folded constants: the same 8*C_out bytes)."""
    b = workload_bytes(wl)
    return fused_bytes(wl) + 3 * b["y"]


def conv_flops(wl) -> int:
    """2 * M * K * C_out with M = N*P*Q and K = kh*kw*C_in (unpadded K)."""
    return 2 * wl.N * wl.P * wl.Q * wl.kh * wl.kw * wl.C_in * wl.C_out


def outputs(wl) -> int:
    return wl.N * wl.P * wl.Q * wl.C_out
