"""The peaks microbenchmark library builds for gfx950 and exports its
launchers (no GPU work here; the GPU run writes profiles/peaks_mi355x.md)."""
import ctypes
import os

from conv2d_batchnorm_silu_amd import peaks


def test_peaks_library_exports():
    path = peaks.LIB if os.path.exists(peaks.LIB) else peaks.build()
    lib = ctypes.CDLL(path)
    for name in ("tgp_copy", "tgp_copy_dma", "tgp_read", "tgp_write", "tgp_mfma", "tgp_mfma_lds", "tgp_valu",
                 "tgp_lds", "tgp_lds_stride", "tgp_lds_pattern", "tgp_vmem_batch"):
        assert getattr(lib, name) is not None
