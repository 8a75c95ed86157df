"""Plain device-to-device copy of a known size, for calibrating HBM counters.

Run under ``rocprofv3 --pmc FETCH_SIZE`` (then ``WRITE_SIZE``): the copy
kernel reads and writes exactly ``--mib`` MiB per dispatch, so the counters'
readings divided by that size give the factor that turns the same counters
of any other kernel into bytes.
"""
from __future__ import annotations

import argparse

import torch


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    n = args.mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {args.mib} MiB x {args.reps}", flush=True)


if __name__ == "__main__":
    main()
