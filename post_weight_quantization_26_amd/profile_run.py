"""Small, fixed workloads to run under rocprofv3.

  python -m post_weight_quantization_26_amd.profile_run copy [--mib 1024]
      One device-to-device copy of a known size (torch's copy kernel). Its
      FETCH_SIZE / WRITE_SIZE counters calibrate what those counters report
      per byte actually moved, so the search kernels' counter readings can be
      converted to HBM bytes.

The search workload itself is profiled through ``bench.py``.
"""
from __future__ import annotations

import argparse
import sys


def copy(mib: int) -> None:
    import torch
    n = mib * (1 << 20) // 2
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB device-to-device", flush=True)


def main(argv=None) -> int:
    p = argparse.ArgumentParser()
    p.add_argument("what", choices=["copy"])
    p.add_argument("--mib", type=int, default=1024)
    a = p.parse_args(argv)
    if a.what == "copy":
        copy(a.mib)
    return 0


if __name__ == "__main__":
    sys.exit(main())
