"""Static checks of the compiled gfx950 code of the kernels that count their
own memory operations (CPU only: hipcc cross-compiles to device assembly).

Several kernels issue direct-to-LDS loads and LDS fragment reads as inline
assembly and wait for them with explicit `s_waitcnt vmcnt(N)` /
`lgkmcnt(N)` counts. Those counts are exact only if the compiler adds no
memory operation of its own that the same counters track: a generic (flat)
access counts on both, and register spills go through scratch memory. Both
have appeared in development after innocent-looking source changes (a
conditional expression over references compiled into a scratch array read
through a flat pointer; a volatile LDS flag compiled into flat loads), so
every build is checked here. Scalar stores are checked as well: the kernels
write memory through vector stores only.
"""
import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

from conv2d_batchnorm_silu_amd import build as B

# Sources whose kernels rely on exact (non-zero) hand-written wait counts.
# (tiled_mfma.hip waits with vmcnt(0)/lgkmcnt(0) only, which any extra
# operation cannot make unsafe.)
COUNTED = ["igemm_cu.hip", "igemm_rw.hip", "igemm_dma.hip", "igemm_patch.hip", "stem.hip"]

FLAT = re.compile(r"^\s*(flat_load|flat_store|flat_atomic|scratch_load|scratch_store)\w*\s")
SCALAR_STORE = re.compile(r"^\s*(s_store|s_buffer_store|s_scratch_store|s_atomic|s_buffer_atomic|"
                          r"s_dcache_wb|s_dcache_discard)\w*\s")
PRIVATE = re.compile(r"\.set\s+(\S+)\.private_seg_size,\s*(\d+)")


def _device_asm(src):
    with tempfile.TemporaryDirectory(prefix="tg_isa_") as d:
        out = os.path.join(d, os.path.basename(src) + ".s")
        cmd = [B.hipcc()] + B.HIPCC_FLAGS + ["--cuda-device-only", "-S", src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, "hipcc failed for %s:\n%s" % (src, r.stderr[-2000:])
        with open(out) as f:
            return f.read()


@pytest.fixture(scope="module")
def listings():
    srcs = [os.path.join(B.CSRC, n) for n in COUNTED]
    with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        return dict(zip(COUNTED, ex.map(_device_asm, srcs)))


def _kernels(asm):
    """Yield (name, body) for every function in a device assembly listing."""
    for m in re.finditer(r"^(_Z\S+):.*?$(.*?)^\.Lfunc_end\d+:", asm, re.M | re.S):
        yield m.group(1), m.group(2)


@pytest.mark.parametrize("src", COUNTED)
def test_no_flat_or_scratch_access(listings, src):
    asm = listings[src]
    found = []
    n = 0
    for name, body in _kernels(asm):
        n += 1
        for line in body.splitlines():
            if FLAT.match(line):
                found.append("%s: %s" % (name[:80], line.strip()))
    assert n > 0, "no kernels found in %s" % src
    assert not found, "flat/scratch accesses break the exact wait counts:\n" + "\n".join(found[:20])


@pytest.mark.parametrize("src", COUNTED)
def test_no_register_spills(listings, src):
    spills = [(k, int(v)) for k, v in PRIVATE.findall(listings[src]) if int(v) != 0]
    assert not spills, "kernels with scratch (spilled registers): %s" % spills[:10]


@pytest.mark.parametrize("src", COUNTED)
def test_no_scalar_stores(listings, src):
    bad = [line.strip() for line in listings[src].splitlines() if SCALAR_STORE.match(line)]
    assert not bad, "scalar memory writes: %s" % bad[:10]


def test_nontemporal_y_stores_kept(listings):
    """The HBM-bound kernels store y with the non-temporal hint (measured:
    plain stores make the 1x1 layer about 25% slower). A store helper that
    took the hint as a run-time flag once let the compiler merge both
    branches into one plain store; every global store of the 1x1 kernel's
    non-temporal instantiations and of the stem kernel must keep `nt`. The
    stem's training-statistics instances (last template argument nonzero) store
    no y, only their per-workgroup statistics, and are not checked."""
    checked = 0
    for src, pat in (("igemm_cu.hip", "igemm_cuILi0ELb1E"), ("stem.hip", "conv2d_bn_silu_stem")):
        for name, body in _kernels(listings[src]):
            if pat not in name:
                continue
            if src == "stem.hip" and "ELi0EEEv" not in name:  # last argument: statistics blocks
                continue
            stores = [l for l in body.splitlines() if l.strip().startswith("global_store")]
            assert stores, name
            plain = [l for l in stores if not l.rstrip().endswith(" nt")]
            assert not plain, "%s: stores without nt:\n%s" % (name, "\n".join(plain[:5]))
            checked += 1
    assert checked >= 4


def test_nontemporal_patch_stores(listings):
    """The patch-staged MFMA kernel writes its output tile once at the end
    with 16-byte (fp16) or 8-byte (fp8) non-temporal stores (measured on the
    3x3 and 7x7 layers: about 3% faster than plain stores); the per-element
    stores of the C_out % 8 != 0 tail may stay plain."""
    checked = 0
    for name, body in _kernels(listings["igemm_patch.hip"]):
        if "conv2d_bn_silu_igemm_patch" not in name:
            continue  # the load-time filter pack kernel
        wide = [l for l in body.splitlines()
                if l.strip().startswith(("global_store_dwordx4", "global_store_dwordx2"))]
        assert wide, name
        plain = [l for l in wide if not l.rstrip().endswith(" nt")]
        assert not plain, "%s: stores without nt:\n%s" % (name, "\n".join(plain[:5]))
        checked += 1
    assert checked >= 10
