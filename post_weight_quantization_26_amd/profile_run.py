"""Small, fixed workloads to run under rocprofv3.

  python -m post_weight_quantization_26_amd.profile_run copy [--mib 1024] [--reps R]
      One device-to-device copy of a known size (torch's copy kernel). Its
      FETCH_SIZE / WRITE_SIZE counters calibrate what those counters report
      per byte actually moved, so the search kernels' counter readings can be
      converted to HBM bytes. With --reps R > 1: R timed copies back to back,
      cycling over enough buffers that no source stays in the last-level
      cache; prints the time per copy (the practical rate of a transfer of
      that size).

  python -m post_weight_quantization_26_amd.profile_run fold [--reps 20]
      The fold of 1/s into a preceding linear layer at the Llama-7B MLP up
      projection size ([11008, 4096] bf16 rows plus bias), in place, ``reps``
      times; prints the average kernel time from the library's HIP-event
      timing and the bandwidth it implies (each element read and written once).

  python -m post_weight_quantization_26_amd.profile_run w4a16 [--reps 20]
      The consumer of the packed layout: the fused GEMV at decode sizes
      (T = 1 and 16 token rows) and the dequantise + MFMA GEMM path at
      T = 4096, on the 4096 x 4096 attention projection and the
      28672 x 8192 70B-class MLP layer (bf16 activations, group 128).
      Prints one JSON line per case with the library's HIP-event kernel times
      and the achieved HBM bandwidth (GEMV) or TFLOP/s (GEMM).

  python -m post_weight_quantization_26_amd.profile_run pack [--reps 20]
      The INT4 g128 pack of a bf16 W with random scales, 28672 x 8192 (the
      70B-class MLP layer) and 4096 x 4096, ``reps`` timed launches each;
      prints the library's HIP-event time and the bandwidth it implies.

  python -m post_weight_quantization_26_amd.profile_run stats [--reps 20]
      The activation statistics (column sums of |x|, then the mean) of a bf16
      X at 65,536 x 4096 (the Llama-7B attention input) and 65,536 x 11,008
      (the MLP down-projection input), ``reps`` timed calls each; prints the
      library's HIP-event time per call and the bandwidth it implies (X read
      once).

  python -m post_weight_quantization_26_amd.profile_run traffic --record R \
          --fetch FETCH.csv --write WRITE.csv
      Updates the traffic record R (profiles/search_gemm_traffic.json or
      profiles/gram_search_traffic.json: kernel, workload, copy calibration
      and the sources it covers) from two rocprofv3 --pmc runs of one
      bench.py step (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch): the
      readings of the record's kernel scaled by the calibration factors give
      its bytes per launch, stored with the SHA-256 of the sources now.

  python -m post_weight_quantization_26_amd.profile_run counters --record R --pmc PMC.csv
      Updates the counter record R (profiles/search_gemm_counters.json or
      profiles/gram_search_counters.json) from one rocprofv3 --pmc run of one
      bench.py step with GRBM_GUI_ACTIVE, SQ_BUSY_CYCLES,
      SQ_VALU_MFMA_BUSY_CYCLES, SQ_LDS_BANK_CONFLICT and SQ_WAVES: the
      record's kernel's readings, its dispatch time under the counters, the
      shader clock they imply (GRBM_GUI_ACTIVE per XCD over the dispatch) and
      the matrix-core utilisation (SQ_VALU_MFMA_BUSY_CYCLES per SIMD over
      GRBM_GUI_ACTIVE per XCD), stored with the SHA-256 of the sources now.

  python -m post_weight_quantization_26_amd.profile_run fused [--reps 3]
      The α search of the 4096 x 4096 bf16 layer over 65,536 tokens and 20
      candidates (INT4, group 128), two-pass (transform writes every
      candidate's E, then the search GEMM) and fused (a parameter pass, then
      the search GEMM forming E itself), ``reps`` timed calls each after one
      warm-up; prints the library's HIP-event kernel times per call and the
      whole call's time, and checks that both curves are identical.

  python -m post_weight_quantization_26_amd.profile_run library_gemm [--reps 5]
      For comparison only: the vendor library's bf16 GEMM (torch.matmul, i.e.
      hipBLASLt) on the search GEMM's shape, X [65536, 4096] times the 20
      candidates' E [81920, 4096] transposed, output [65536, 81920] bf16;
      prints its time and TFLOP/s (torch events on the current stream).

The search workload itself is profiled through ``bench.py``.
"""
from __future__ import annotations

import argparse
import sys


def copy(mib: int, reps: int = 1) -> None:
    import torch
    n = mib * (1 << 20) // 2
    if reps <= 1:
        src = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copied {mib} MiB device-to-device", flush=True)
        return
    # timed copies cycling over enough buffers (at least 512 MiB of sources)
    # that no source stays in the 256 MB last-level cache between its uses
    import json
    nbuf = max(2, -(-512 // mib))
    bufs = [(torch.empty(n, dtype=torch.bfloat16, device="cuda:0").fill_(1.0),
             torch.empty(n, dtype=torch.bfloat16, device="cuda:0")) for _ in range(nbuf)]
    for s_, d_ in bufs:
        d_.copy_(s_)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        s_, d_ = bufs[i % nbuf]
        d_.copy_(s_)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    moved = 2 * n * 2
    print(json.dumps({"copy_mib": mib, "reps": reps, "buffers": nbuf, "us_per_copy": round(us, 2),
                      "GBps_read_plus_write": round(moved / (us * 1e-6) / 1e9, 1)}), flush=True)


def fill(mib: int, reps: int) -> None:
    """Write-only rate: torch's fill of a mib-MiB bf16 buffer, reps times."""
    import json
    import torch
    x = torch.empty(mib * (1 << 20) // 2, dtype=torch.bfloat16, device="cuda:0")
    for _ in range(3):
        x.fill_(1.0)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        x.fill_(1.0)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    print(json.dumps({"fill_mib": mib, "reps": reps, "us_per_fill": round(us, 2),
                      "GBps_written": round(mib * (1 << 20) / (us * 1e-6) / 1e9, 1)}), flush=True)


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


def w4a16(reps: int) -> None:
    import json
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import torch
    from post_weight_quantization_26_amd import api
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    for N, K, bits in ((4096, 4096, 4), (28672, 8192, 4), (4096, 4096, 3), (28672, 8192, 3)):
        W = (torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        s = torch.ones(K, dtype=torch.float32, device=dev)
        qw, qz, sc = api.quantize_pack(W, s, bits=bits)
        del W
        for T in (1, 4, 16, 4096):
            X = torch.randn((T, K), generator=g, device=dev).to(torch.bfloat16)
            need = (api.w4a16_workspace_bytes if bits == 4 else api.w3a16_workspace_bytes)(
                T, N, K, torch.bfloat16)
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            Y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
            n_rep = reps if T <= 16 else max(3, reps // 4)
            api.w4a16_matmul(X, qw, qz, sc, ws=ws, out=Y, bits=bits)
            torch.cuda.synchronize()
            api.profile_enable(True)
            api.profile_reset()
            for _ in range(n_rep):
                api.w4a16_matmul(X, qw, qz, sc, ws=ws, out=Y, bits=bits)
            torch.cuda.synchronize()
            t = {k: api.profile_read(k) for k in ("dequant", "w4a16", "w4a16_reduce")}
            api.profile_enable(False)
            main_us = t["w4a16"][0] * 1e3 / n_rep
            rec = {"N": N, "K": K, "T": T, "bits": bits, "main_kernel_us": round(main_us, 2)}
            packed = N * K * bits // 8 + (N * K // 128) * (2 + bits / 8)
            if T <= 16:
                # what any decode kernel must move: the packed layer, X and Y
                moved = packed + T * K * 2 + T * N * 2
                rec.update(path="gemv", reduce_us=round(t["w4a16_reduce"][0] * 1e3 / n_rep, 2),
                           algorithmic_bytes=int(moved),
                           GBps=round(moved / (main_us * 1e-6) / 1e9, 1),
                           frac_of_8TBps=round(moved / (main_us * 1e-6) / 8e12, 4))
            else:
                flops = 2.0 * T * N * K
                rec.update(path="gemm", dequant_us=round(t["dequant"][0] * 1e3 / n_rep, 2),
                           TFLOPs=round(flops / (main_us * 1e-6) / 1e12, 1),
                           frac_of_2500=round(flops / (main_us * 1e-6) / 2.5e15, 4))
            print(json.dumps(rec), flush=True)
            if T > 16 and bits == 4:
                # the GEMM that dequantises on the fly (no workspace)
                api.w4a16_matmul(X, qw, qz, sc, out=Y, on_the_fly=True)
                torch.cuda.synchronize()
                api.profile_enable(True)
                api.profile_reset()
                for _ in range(n_rep):
                    api.w4a16_matmul(X, qw, qz, sc, out=Y, on_the_fly=True)
                torch.cuda.synchronize()
                fly_us = api.profile_read("w4a16")[0] * 1e3 / n_rep
                api.profile_enable(False)
                print(json.dumps({"N": N, "K": K, "T": T, "bits": bits,
                                  "main_kernel_us": round(fly_us, 2), "path": "gemm_on_the_fly",
                                  "TFLOPs": round(flops / (fly_us * 1e-6) / 1e12, 1),
                                  "frac_of_2500": round(flops / (fly_us * 1e-6) / 2.5e15, 4)}),
                      flush=True)
            del X, ws, Y
        del qw, qz, sc
        torch.cuda.empty_cache()


def pack(reps: int) -> None:
    import json
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import torch
    from post_weight_quantization_26_amd import api
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    for N, K in ((28672, 8192), (4096, 4096)):
        W = (torch.randn((N, K), generator=g, device=dev) * 0.015).to(torch.bfloat16)
        s = torch.exp(torch.rand(K, generator=g, device=dev) * 2 - 1)
        out = api.quantize_pack(W, s)
        torch.cuda.synchronize()
        api.profile_enable(True)
        api.profile_reset()
        for _ in range(reps):
            api.quantize_pack(W, s, out=out)
        torch.cuda.synchronize()
        ms, n = api.profile_read("pack")
        api.profile_enable(False)
        us = ms / n * 1e3
        moved = N * K * 2 + N * K // 2 + (N * K // 128) * 2.5 + K * 4
        print(json.dumps({"N": N, "K": K, "pack_us": round(us, 2), "algorithmic_bytes": int(moved),
                          "GBps": round(moved / (us * 1e-6) / 1e9, 1)}), flush=True)
        del W, out
        torch.cuda.empty_cache()


def stats(reps: int) -> None:
    import json
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import torch
    from post_weight_quantization_26_amd import _lib, api
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    for T, K in ((65536, 4096), (65536, 11008)):
        X = torch.randn((T, K), generator=g, device=dev).to(torch.bfloat16)
        ws = torch.empty(api.workspace_bytes(_lib.AWQ_OP_STATS, T, 1, K, 1, X.dtype),
                         dtype=torch.uint8, device=dev)
        out = api.act_stats(X, ws=ws)
        torch.cuda.synchronize()
        api.profile_enable(True)
        api.profile_reset()
        for _ in range(reps):
            api.act_stats(X, ws=ws, out=out)
        torch.cuda.synchronize()
        ms, n = api.profile_read("stats")
        api.profile_enable(False)
        us = ms / n * 1e3
        moved = T * K * 2
        print(json.dumps({"T": T, "K": K, "stats_us": round(us, 2), "algorithmic_bytes": moved,
                          "GBps": round(moved / (us * 1e-6) / 1e9, 1)}), flush=True)
        del X, ws, out
        torch.cuda.empty_cache()


def traffic(record: str, fetch_csv: str, write_csv: str) -> None:
    import csv
    import hashlib
    import json
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    with open(record) as f:
        rec = json.load(f)

    def reading(path: str, counter: str) -> float:
        vals = []
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row["Kernel_Name"]
                if row["Counter_Name"] == counter and f"::{rec['kernel']}(" in name:
                    vals.append(float(row["Counter_Value"]))
        if len(vals) != 1:
            raise SystemExit(f"{path}: expected one {rec['kernel']} dispatch, found {len(vals)}")
        return vals[0]

    cal = rec["copy_calibration"]
    fetch_kb = reading(fetch_csv, "FETCH_SIZE")
    write_kb = reading(write_csv, "WRITE_SIZE")
    rec["fetch_size_kb"] = fetch_kb
    rec["write_size_kb"] = write_kb
    rec["bytes_per_launch"] = int(round(fetch_kb * 1024 * cal["fetch_factor"]
                                        + write_kb * 1024 * cal["write_factor"]))
    h = hashlib.sha256()
    for rel in rec["gemm_sources"]:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    rec["gemm_sources_sha256"] = h.hexdigest()
    with open(record, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps({"kernel": rec["kernel"], "fetch_size_kb": fetch_kb, "write_size_kb": write_kb,
                      "GiB_per_launch": round(rec["bytes_per_launch"] / 2 ** 30, 2)}))


XCDS, SIMDS = 8, 1024   # MI355X: 8 XCDs, 256 CUs of 4 SIMDs


def counters(record: str, pmc_csv: str) -> None:
    import csv
    import hashlib
    import json
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    with open(record) as f:
        rec = json.load(f)
    vals, span = {}, None
    with open(pmc_csv) as f:
        for row in csv.DictReader(f):
            if f"::{rec['kernel']}(" not in row["Kernel_Name"]:
                continue
            key = (row["Dispatch_Id"], row["Counter_Name"])
            vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
            span = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9
    dispatches = {d for d, _ in vals}
    if len(dispatches) != 1:
        raise SystemExit(f"{pmc_csv}: expected one {rec['kernel']} dispatch, found {len(dispatches)}")
    rd = {c: v for (_, c), v in vals.items()}
    gui = rd["GRBM_GUI_ACTIVE"] / XCDS
    rec["counters"] = rd
    rec["dispatch_us_under_counters"] = round(span * 1e6, 1)
    rec["clock_ghz"] = round(gui / span / 1e9, 3)
    rec["mfma_busy_frac"] = round(rd["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS / gui, 4)
    h = hashlib.sha256()
    for rel in rec["gemm_sources"]:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    rec["gemm_sources_sha256"] = h.hexdigest()
    with open(record, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps({"kernel": rec["kernel"], "clock_ghz": rec["clock_ghz"],
                      "mfma_busy_frac": rec["mfma_busy_frac"]}))


def library_gemm(reps: int) -> None:
    import json
    import torch
    T, K, Nc = 65536, 4096, 20 * 4096
    g = torch.Generator(device="cuda:0")
    g.manual_seed(11)
    X = torch.randn((T, K), generator=g, device="cuda:0").to(torch.bfloat16)
    E = (torch.randn((Nc, K), generator=g, device="cuda:0") * 1e-3).to(torch.bfloat16)
    Y = torch.empty((T, Nc), dtype=torch.bfloat16, device="cuda:0")
    for _ in range(2):
        torch.matmul(X, E.t(), out=Y)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        torch.matmul(X, E.t(), out=Y)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    flops = 2.0 * T * Nc * K
    print(json.dumps({"op": "torch.matmul bf16 X·Eᵀ", "T": T, "Nc": Nc, "K": K, "ms": round(ms, 3),
                      "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
                      "frac_of_2500": round(flops / (ms * 1e-3) / 2.5e15, 4)}), flush=True)


def fused(reps: int) -> None:
    import json
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import numpy as np
    import torch
    from post_weight_quantization_26_amd import api
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    T, N, K = 65536, 4096, 4096
    X = torch.randn((T, K), generator=g, device=dev)
    X[:, :41] *= 20.0   # a few large input channels
    X = X.to(torch.bfloat16)
    W = (torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    abar = api.act_stats(X)
    alphas = [i / 20 for i in range(20)]
    ws = torch.empty(api.workspace_bytes(api.L.AWQ_OP_SEARCH_SCALE, T, N, K, 20, X.dtype),
                     dtype=torch.uint8, device=dev)
    curves = {}
    for fz in (False, True):
        api.search_scale(X, W, abar, alphas, ws=ws, fused=fz)
        torch.cuda.synchronize()
        api.profile_enable(True)
        api.profile_reset()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            r = api.search_scale(X, W, abar, alphas, ws=ws, fused=fz)
        b.record()
        torch.cuda.synchronize()
        t = {k: api.profile_read(k)[0] / reps for k in ("transform", "gemm", "reduce")}
        api.profile_enable(False)
        curves[fz] = r["mse"]
        flops = 2.0 * T * 20 * N * K
        print(json.dumps({"path": "fused" if fz else "two-pass",
                          "transform_or_params_ms": round(t["transform"], 3),
                          "gemm_ms": round(t["gemm"], 3), "reduce_ms": round(t["reduce"], 3),
                          "call_ms": round(a.elapsed_time(b) / reps, 3),
                          "gemm_frac_of_2500": round(flops / (t["gemm"] * 1e-3) / 2.5e15, 4)}),
              flush=True)
    print(json.dumps({"curves_identical": bool(np.array_equal(curves[False], curves[True]))}),
          flush=True)


def main(argv=None) -> int:
    p = argparse.ArgumentParser()
    p.add_argument("what", choices=["copy", "fill", "fold", "w4a16", "pack", "stats", "traffic",
                                    "counters", "library_gemm", "fused"])
    p.add_argument("--pmc")
    p.add_argument("--mib", type=int, default=1024)
    p.add_argument("--reps", type=int, default=20)
    p.add_argument("--record")
    p.add_argument("--fetch")
    p.add_argument("--write")
    a = p.parse_args(argv)
    if a.what == "traffic":
        traffic(a.record, a.fetch, a.write)
    elif a.what == "counters":
        counters(a.record, a.pmc)
    elif a.what == "library_gemm":
        library_gemm(a.reps)
    elif a.what == "fused":
        fused(a.reps if a.reps != 20 else 3)
    elif a.what == "copy":
        copy(a.mib, a.reps if a.reps != 20 else 1)
    elif a.what == "fill":
        fill(a.mib, a.reps)
    elif a.what == "fold":
        fold(a.reps)
    elif a.what == "pack":
        pack(a.reps)
    elif a.what == "stats":
        stats(a.reps)
    else:
        w4a16(a.reps)
    return 0


if __name__ == "__main__":
    sys.exit(main())
