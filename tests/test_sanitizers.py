"""CPU sanitizer builds: AddressSanitizer and UndefinedBehaviorSanitizer on
the oracle (oracle/oracle.c, built with gcc) and on the host side of the C ABI
(api.hip, built with hipcc with the sanitizers on the host pass only, linked
against the library's other objects through libtgconv.so). Each build runs a
driver under tests/sanitize/ that exercises the entry points without a GPU;
any memory or undefined-behaviour error aborts the driver, which fails the
test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
PKG = os.path.join(ROOT, "conv2d_batchnorm_silu_amd")
ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-std=c99", "-Wall",
          "-o", exe, os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
          "-lm", "-lpthread"])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1"))
    assert "0 failures" in r.stdout, r.stdout


def test_host_abi_under_asan_ubsan(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    lib = os.path.join(PKG, "libtgconv.so")
    if not os.path.exists(hipcc) or not os.path.exists(lib):
        pytest.skip("hipcc or the built library not available")
    from conv2d_batchnorm_silu_amd.build import ARCH, HIPCC_FLAGS
    obj = str(tmp_path / "api_san.o")
    flags = [f for f in HIPCC_FLAGS if f != "-O3"]
    _run([hipcc] + flags + ["-O1", "-g", "-fno-omit-frame-pointer",
                            "-Xarch_host", "-fsanitize=address",
                            "-Xarch_host", "-fsanitize=undefined",
                            "-Xarch_host", "-fno-sanitize-recover=all",
                            "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", obj])
    exe = str(tmp_path / "abi_driver")
    _run([hipcc, "--offload-arch=" + ARCH, "-g",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-I", os.path.join(ROOT, "include"), "-x", "c", os.path.join(SAN, "abi_driver.c"),
          "-x", "none", obj, "-L", PKG, "-ltgconv", "-Wl,-rpath," + PKG, "-o", exe])
    r = _run([exe], env=ENV)
    assert "0 failures" in r.stdout, r.stdout
