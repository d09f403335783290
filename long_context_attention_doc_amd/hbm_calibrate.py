"""Plain device-to-device copy of a known size, for calibrating HBM counters.

Run under a counter profiler, e.g.
  rocprofv3 --pmc FETCH_SIZE -- python3 -m long_context_attention_doc_amd.hbm_calibrate
The copy kernel reads and writes exactly `--mib` MiB per launch, so the
profiler's FETCH_SIZE / WRITE_SIZE for it give the scale between those
counters and bytes moved.
"""
import argparse

import torch


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    a = ap.parse_args()
    n = a.mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(a.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {a.mib} MiB x {a.reps}")


if __name__ == "__main__":
    main()
