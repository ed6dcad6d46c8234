"""Calibration run for rocprofv3's HBM byte counters.

Copies a device buffer of known size a few times with a plain device-to-device
copy, so that the FETCH_SIZE and WRITE_SIZE readings of that copy kernel
(exactly `bytes` read and `bytes` written per dispatch) give the scale from
counter units to HBM bytes. Run under rocprofv3 --pmc; prints one JSON line.
"""

from __future__ import annotations

import argparse
import json

import torch


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=512, help="buffer size in MiB")
    ap.add_argument("--copies", type=int, default=3)
    args = ap.parse_args()
    n = args.mib << 20
    dev = torch.device("cuda:0")
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.copies):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"bytes_per_copy": n, "copies": args.copies}))


if __name__ == "__main__":
    main()
