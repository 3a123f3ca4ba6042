"""Plain device copy of a known size, for calibrating HBM traffic counters.

python -m moe_measure.hbm_copy_probe [--mib 1024] [--reps 3]

Copies a --mib MiB buffer into another with torch's copy kernel --reps
times.  Under `rocprofv3 --pmc FETCH_SIZE` (then WRITE_SIZE) each copy
dispatch should read (write) exactly that many bytes; the ratio between the
known size and the counter reading is the scale applied to the counters of
the MoE kernels.
"""

import argparse

import torch


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args(argv)
    n = args.mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {args.mib} MiB x {args.reps}", flush=True)


if __name__ == "__main__":
    main()
