"""Build libtgconv.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each source compiles to its own object in parallel, then one link step makes
the shared library next to this file. Run ``python -m
conv2d_batchnorm_silu_amd.build`` or ``__graft_entry__.build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libtgconv.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

# Packed FP32 instructions are switched off for all device code: the compiler
# would otherwise form them from ordinary float arithmetic.
# MFMA results are kept in ordinary VGPRs (gfx950 MFMA may write either file):
# the epilogue then reads its accumulators without one v_accvgpr_read per
# value, which is a sixth of the fused epilogue's VALU work.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form",
               "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtgconv.so)")


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, extra: list) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + HIPCC_FLAGS + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build_library(extra_flags: list | None = None, jobs: int | None = None) -> str:
    """Compile every csrc/*.hip and link libtgconv.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra_flags or [])
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=jobs or min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library())
