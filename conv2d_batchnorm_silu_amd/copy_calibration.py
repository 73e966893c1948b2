"""Plain device copy of known size, for calibrating rocprofv3's FETCH_SIZE and
WRITE_SIZE counters: each copy reads and writes exactly COPY_BYTES.

Run under ``rocprofv3 --pmc FETCH_SIZE`` (and separately ``WRITE_SIZE``); the
counter value per copy dispatch divided by COPY_BYTES is the scale factor
applied to the fused kernel's counters. ``--dma`` copies with this library's
own kernel that reads through direct-to-LDS buffer loads (peaks.hip,
pk_copy_dma), the way the fused kernels read x; without it, torch's copy.
``--rotate`` spreads the copies over SETS buffer pairs.
"""
import sys

import torch

COPY_BYTES = 256 * 2**20
REPS = 5
SETS = 4


def main():
    # Default: torch's copy of one buffer pair, REPS times. --dma: this
    # library's copy that reads through direct-to-LDS buffer loads. --rotate:
    # each copy takes the next of SETS buffer pairs (no reuse between copies).
    args = sys.argv[1:]
    sets = SETS if "--rotate" in args else 1
    a = [torch.full((COPY_BYTES // 2,), float(k + 1), dtype=torch.float16, device="cuda")
         for k in range(sets)]
    b = [torch.empty_like(t) for t in a]
    if "--dma" in args:
        import os
        sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
        from conv2d_batchnorm_silu_amd import peaks
        lib = peaks._lib()
        s = torch.cuda.current_stream().cuda_stream
        for r in range(REPS):
            k = r % sets
            assert lib.tgp_copy_dma(a[k].data_ptr(), b[k].data_ptr(), COPY_BYTES, 2048, s) == 0
    else:
        for r in range(REPS):
            b[r % sets].copy_(a[r % sets])
    torch.cuda.synchronize()
    for k in range(min(sets, REPS)):
        assert torch.equal(a[k], b[k])
    print("copied %d x %d bytes" % (REPS, COPY_BYTES))


if __name__ == "__main__":
    main()
