"""Small, fixed workloads to run under rocprofv3.

  python -m post_weight_quantization_26_amd.profile_run copy [--mib 1024]
      One device-to-device copy of a known size (torch's copy kernel). Its
      FETCH_SIZE / WRITE_SIZE counters calibrate what those counters report
      per byte actually moved, so the search kernels' counter readings can be
      converted to HBM bytes.

  python -m post_weight_quantization_26_amd.profile_run fold [--reps 20]
      The fold of 1/s into a preceding linear layer at the Llama-7B MLP up
      projection size ([11008, 4096] bf16 rows plus bias), in place, ``reps``
      times; prints the average kernel time from the library's HIP-event
      timing and the bandwidth it implies (each element read and written once).

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


def fold(reps: int) -> None:
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import numpy as np
    import torch
    from post_weight_quantization_26_amd import api, synth
    K, K_prev = 11008, 4096
    W = synth.make_weight(K, K_prev, 0.02, "bf16", cid=3)
    Wd = torch.from_numpy(W.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    bias = torch.zeros(K, dtype=torch.bfloat16, device="cuda:0")
    # s of alternating 2 and 1/2: exact in bf16, so repeated folds stay finite
    s = torch.from_numpy(np.where(np.arange(K) % 2 == 0, 2.0, 0.5).astype(np.float32)).to("cuda:0")
    api.fold_linear(Wd, s, bias)
    torch.cuda.synchronize()
    api.profile_enable(True)
    api.profile_reset()
    for _ in range(reps):
        api.fold_linear(Wd, s, bias)
    torch.cuda.synchronize()
    ms, n = api.profile_read("fold")
    api.profile_enable(False)
    rows_ms = ms / reps   # per fold_linear call: rows kernel + bias kernel
    moved = 2 * (K * K_prev * 2 + K * 2)
    print(f"fold_linear [{K}, {K_prev}] bf16 + bias: {rows_ms * 1e3:.1f} us per call "
          f"({n // reps} launches), {moved / (rows_ms / 1e3) / 1e9:.0f} GB/s", flush=True)


def main(argv=None) -> int:
    p = argparse.ArgumentParser()
    p.add_argument("what", choices=["copy", "fold"])
    p.add_argument("--mib", type=int, default=1024)
    p.add_argument("--reps", type=int, default=20)
    a = p.parse_args(argv)
    if a.what == "copy":
        copy(a.mib)
    else:
        fold(a.reps)
    return 0


if __name__ == "__main__":
    sys.exit(main())
