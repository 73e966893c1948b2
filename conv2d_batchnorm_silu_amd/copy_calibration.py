"""Plain device copy of known size, for calibrating rocprofv3's FETCH_SIZE and
WRITE_SIZE counters: each copy reads and writes exactly COPY_BYTES.

Run under ``rocprofv3 --pmc FETCH_SIZE`` (and separately ``WRITE_SIZE``); the
counter value per copy dispatch divided by COPY_BYTES is the scale factor
applied to the fused kernel's counters.
"""
import torch

COPY_BYTES = 256 * 2**20
REPS = 5


def main():
    a = torch.empty(COPY_BYTES // 2, dtype=torch.float16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(REPS):
        b.copy_(a)
    torch.cuda.synchronize()
    print("copied %d x %d bytes" % (REPS, COPY_BYTES))


if __name__ == "__main__":
    main()
