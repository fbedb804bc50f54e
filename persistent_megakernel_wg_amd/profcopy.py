"""Calibration run for HBM traffic counters: a plain device copy of known size.

    python -m persistent_megakernel_wg_amd.profcopy [--mib 1024] [--reps 3]

Under `rocprofv3 --pmc FETCH_SIZE` (or WRITE_SIZE) each copy dispatch reads
(writes) exactly MiB * 1024 KiB; the ratio of that to what the counter reports
scales the megakernel's counter readings to bytes.
"""
from __future__ import annotations

import argparse


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    import torch
    n = args.mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("copied %d MiB x %d" % (args.mib, args.reps), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
