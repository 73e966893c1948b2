"""Fused conv2d + BatchNorm + SiLU for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library (``libtgconv.so``, built from
``csrc/``) of hand-written HIP kernels; ``binding`` wraps it with ctypes and
uses PyTorch only for device memory and streams. ``inputs`` holds the seeded
synthetic data recipes shared by tests and the benchmark.

Importing this package does not load the shared library; the first use of a
binding name does, and fails loudly if the library is missing.
"""
from __future__ import annotations

_BINDING_NAMES = {
    "ConvBnSilu", "bn_fold", "library", "Kernel", "Dtype", "TgError", "status_string",
    "kernel_name", "library_path", "build_library", "exported_symbols", "Table", "dispatch_choose",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
