"""Benchmark: AWQ per-layer search throughput on one MI355X.

A step is one pass of the whole per-layer path over one synthetic layer
already resident in HBM: activation statistics, the scale table and the
α-grid search (quantise / dequantise / fold candidates, the search GEMM with
its squared-error epilogue, reductions, argmin), the clip search when the
workload has one, and INT4 packing. The default workload is a Llama-7B-shaped
attention projection: W [4096, 4096] bf16, X [65536, 4096] bf16 with 41
outlier channels, INT4 asymmetric g128, 20 α values, then pack.

Prints one JSON line. ``value`` is α-candidates evaluated per second over the
timed steps (whole job). ``roofline`` covers the dominant kernel, the search
GEMM, timed with HIP events on its launch stream inside the timed region.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 and fp16 MFMA, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published (the float32 search GEMM uses FMAs)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
TRAFFIC_FILES = {"direct": os.path.join(ROOT, "profiles", "search_gemm_traffic.json"),
                 "gram": os.path.join(ROOT, "profiles", "gram_search_traffic.json")}
COUNTER_FILES = {"direct": os.path.join(ROOT, "profiles", "search_gemm_counters.json"),
                 "gram": os.path.join(ROOT, "profiles", "gram_search_counters.json")}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--config", default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=2048)
    p.add_argument("--method", choices=["direct", "gram"], default="direct",
                   help="candidate errors as X·Eᵀ (direct) or E·G·Eᵀ with G = XᵀX (gram)")
    p.add_argument("--no-gram", action="store_true",
                   help="skip the second measurement through the Gram path")
    return p.parse_args()


def _current_record(path: str, cfg_name: str):
    """A committed counter record, or None when the kernel source changed
    since its counters were taken or it covers another workload."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for rel in rec.get("gemm_sources", []):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    if rec.get("gemm_sources_sha256") != h.hexdigest() or rec.get("workload") != cfg_name:
        return None
    return rec


def gemm_traffic(cfg_name: str, how: str = "direct"):
    """HBM bytes per launch of the candidate GEMM (search GEMM, or the Gram
    search) from committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs, or None."""
    rec = _current_record(TRAFFIC_FILES[how], cfg_name)
    return None if rec is None else rec.get("bytes_per_launch")


def gemm_mfma_util(cfg_name: str, how: str = "direct"):
    """Matrix-core utilisation of the candidate GEMM from a committed rocprofv3
    counter run (SQ_VALU_MFMA_BUSY_CYCLES per SIMD over GRBM_GUI_ACTIVE per
    XCD, in that run's own dispatch), with the shader clock it ran at; None
    when stale."""
    rec = _current_record(COUNTER_FILES[how], cfg_name)
    if rec is None:
        return None
    return {"frac": rec["mfma_busy_frac"], "clock_ghz": rec["clock_ghz"],
            "dispatch_us_under_counters": rec["dispatch_us_under_counters"],
            "source": os.path.relpath(COUNTER_FILES[how], ROOT)}


def host_cpu():
    """The host's CPU model, physical cores and logical CPUs, from lscpu."""
    import subprocess
    info = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            info[k.strip()] = v.strip()
    except Exception:  # pragma: no cover
        pass

    def num(key):
        try:
            return int(info.get(key, ""))
        except ValueError:
            return None
    cps, sockets = num("Core(s) per socket"), num("Socket(s)")
    return {"model": info.get("Model name"),
            "physical_cores": cps * sockets if cps and sockets else None,
            "logical_cpus": num("CPU(s)") or os.cpu_count()}


def cpu_baseline(cfg, X, Ws, alphas, rows_n: int):
    """The CPU oracle, as it stands, on a bounded sample of one step: stats over
    the full X, the α search over ``rows_n`` evenly spaced output rows (all
    tokens, all α; extrapolated linearly to N rows, since every row costs the
    same), and packing of every full W. ``Ws`` holds one layer, or the layers
    of a group that share X (searched together, with the fold into the
    normalisation timed too)."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    rows = np.unique(np.linspace(0, cfg.N - 1, rows_n).round().astype(np.int64))
    t0 = time.perf_counter()
    ab = O.act_stats(X, cfg.dtype)
    t1 = time.perf_counter()
    res = O.search_scale_group(X, Ws, cfg.dtype, ab, alphas, cfg.bits, cfg.group,
                               cfg.zero_point, rows=rows)
    t2 = time.perf_counter()
    if cfg.layers:
        from post_weight_quantization_26_amd import synth
        O.fold_norm(synth.make_norm_weight(cfg.K, cfg.dtype, cid=cfg.cid)[0], None, cfg.dtype,
                    res["s_best"])
    if cfg.pack:
        for W in Ws:
            O.quantize_pack(W, cfg.dtype, res["s_best"], None, cfg.bits, cfg.group,
                            cfg.zero_point)
    pack_t = time.perf_counter() - t2
    step = (t1 - t0) + (t2 - t1) * cfg.N / len(rows) + pack_t
    return {"value": len(alphas) / step, "unit": "alpha-candidates/s", "cores": int(threads),
            "kind": "oracle", "host": host_cpu(),
            "sample": (f"stats over all {cfg.T} tokens; alpha search over {len(rows)} of {cfg.N} "
                       f"output rows (all {len(alphas)} alphas, all tokens) extrapolated x"
                       f"{cfg.N / len(rows):.0f}" + ("; fold into the norm weight" if cfg.layers
                                                     else "")
                       + ("; pack of every full W" if cfg.pack else "")),
            "sample_seconds": round(time.perf_counter() - t0, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    from post_weight_quantization_26_amd import build_lib, synth
    if not os.path.exists(build_lib.LIB_PATH):
        build_lib.build()
    from post_weight_quantization_26_amd import _lib, api

    name = args.config or synth.BENCH_CONFIG
    cfg = synth.CONFIGS[name]
    dev = torch.device("cuda:0")
    if cfg.layers:
        X, Ws = synth.make_group(cfg)
    else:
        X, W = synth.make_layer(cfg)
        Ws = [W]
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(cfg.dtype, torch.float32)

    def up(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        if cfg.dtype == "f16":
            return torch.from_numpy(a.view(np.float16)).to(dev)
        return torch.from_numpy(a).to(dev)

    Xd = up(X)
    Wds = [up(W) for W in Ws]
    gamma = up(synth.make_norm_weight(cfg.K, cfg.dtype, cid=cfg.cid)[0]) if cfg.layers else None
    alphas = synth.alpha_grid(cfg.n_alpha)
    ratios = synth.ratio_grid(cfg.n_ratio) if cfg.n_ratio else None
    T, N, K = cfg.T, cfg.N, cfg.K
    ws_stats = torch.empty(api.workspace_bytes(_lib.AWQ_OP_STATS, T, 1, K, 1, tdt),
                           dtype=torch.uint8, device=dev)
    n_grid = max(cfg.n_alpha, cfg.n_ratio)
    method = args.method
    gram_ok = cfg.dtype == "bf16"
    if method == "gram" and not gram_ok:
        print(json.dumps({"error": "the Gram path runs bf16 layers"}))
        sys.exit(2)
    ws_need = api.workspace_bytes(_lib.AWQ_OP_SEARCH_SCALE, T, N, K, n_grid, tdt)
    if gram_ok:
        ws_need = max(ws_need, api.workspace_bytes(_lib.AWQ_OP_SEARCH_SCALE_GRAM, T, N, K, n_grid,
                                                   tdt))
    ws_search = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    if gram_ok:
        # the Gram path builds G once per step and shares it among the searches
        G_buf = torch.empty(api.gram_bytes(K), dtype=torch.uint8, device=dev)
        ws_gram = torch.empty(api.workspace_bytes(_lib.AWQ_OP_GRAM_BUILD, T, 1, K, 1, tdt),
                              dtype=torch.uint8, device=dev)
    ws_pack = torch.empty(256, dtype=torch.uint8, device=dev)
    abar = torch.empty(K, dtype=torch.float32, device=dev)
    G = cfg.group
    pack_out = [(torch.empty((K, Wd.shape[0] * cfg.bits // 32), dtype=torch.int32, device=dev),
                 torch.empty((K // G, Wd.shape[0] * cfg.bits // 32), dtype=torch.int32, device=dev),
                 torch.empty((K // G, Wd.shape[0]), dtype=torch.float16, device=dev))
                for Wd in Wds]
    zp = cfg.zero_point
    cands_per_step = cfg.n_alpha + (cfg.n_ratio or 0)   # clip candidates: per layer, N rows in all

    def step(how):
        api.act_stats(Xd, ws=ws_stats, out=abar)
        Gm = api.gram_build(Xd, ws=ws_gram, out=G_buf) if how == "gram" else None
        if cfg.layers:
            # linears sharing X: one search, one s, folded into the norm weight
            # (in place, so gamma drifts over the steps; the work is the same)
            res = api.search_scale_group(Xd, Wds, abar, alphas, bits=cfg.bits, group=G,
                                         zero_point=zp, ws=ws_search, method=how, G=Gm)
            api.fold_norm(gamma, res["s_best"])
        else:
            res = api.search_scale(Xd, Wds[0], abar, alphas, bits=cfg.bits, group=G,
                                   zero_point=zp, ws=ws_search, method=how, G=Gm)
        for Wd, out in zip(Wds, pack_out):
            ratio = None
            if ratios is not None:
                ratio = api.search_clip(Xd, Wd, res["s_best"], ratios, bits=cfg.bits, group=G,
                                        zero_point=zp, ws=ws_search, method=how,
                                        G=Gm)["ratio_best"]
            if cfg.pack:
                api.quantize_pack(Wd, res["s_best"], ratio, bits=cfg.bits, group=G, zero_point=zp,
                                  ws=ws_pack, out=out)
        return res

    def measure(how):
        """Warm-up, then exactly args.steps timed steps between synchronisations;
        kernel times from the library's HIP events on the launch stream."""
        for _ in range(args.warmup):
            step(how)
        torch.cuda.synchronize()
        api.profile_enable(True)
        api.profile_reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            res = step(how)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        prof = {k: api.profile_read(k) for k in _lib.KERNEL_KINDS}
        api.profile_enable(False)
        elapsed = t1 - t0
        if how == "gram":
            # hi and lo halves of G' (diagonal 256-tiles of G, tiles above it
            # doubled) against each candidate row: row tile tm contracts over
            # K - 256·tm columns, 2·2·Σ_tm rows_tm·(K - 256·tm) flops per row
            gemm_ms, gemm_n = prof["gram_search"]
            tri = sum(min(256, K - m0) * (K - m0) for m0 in range(0, K, 256))
            flops_per_step = 2.0 * 2 * tri * N * cands_per_step
            kernel_name = "gram_search_kernel"
        else:
            gemm_ms, gemm_n = prof["gemm"]
            flops_per_step = 2.0 * T * N * K * cands_per_step
            kernel_name = {"bf16": "search_gemm_bf16_kernel", "f16": "search_gemm_f16_kernel"}.get(
                cfg.dtype, "search_gemm_f32_kernel")
        gemm_avg_s = gemm_ms / 1e3 / max(gemm_n, 1)
        launches_per_step = gemm_n // args.steps if args.steps else 0
        flops_per_launch = flops_per_step / max(launches_per_step, 1)
        achieved = flops_per_launch / gemm_avg_s / 1e12
        traffic = gemm_traffic(name, how)
        f32 = cfg.dtype == "f32"
        peak = FP32_VECTOR_PEAK_TFLOPS if f32 else MFMA_BF16_PEAK_TFLOPS
        roof = {"bound": "alu" if f32 else "mfma", "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4),
                "traffic": traffic, "kernel": kernel_name,
                "avg_launch_us": round(gemm_avg_s * 1e6, 1),
                "algorithmic_flops_per_launch": flops_per_launch,
                "mfma_util_counters": None if f32 else gemm_mfma_util(name, how)}
        kernels = {k: {"avg_us": round(ms * 1e3 / n, 2) if n else None, "launches": n,
                       "share_of_step": round(ms / (elapsed * 1e3), 4)}
                   for k, (ms, n) in prof.items() if n}
        return elapsed, prof, res, roof, kernels

    elapsed, prof, res, roofline, kernels = measure(method)
    value = cfg.n_alpha * args.steps / elapsed
    achieved = roofline["achieved"]
    other = None
    if method == "direct" and gram_ok and not args.no_gram:
        g_el, _, g_res, g_roof, g_kern = measure("gram")
        other = {"method": "gram", "value": round(cfg.n_alpha * args.steps / g_el, 3),
                 "all_candidates_per_s": round(cands_per_step * args.steps / g_el, 3),
                 "ms_per_step": round(g_el / args.steps * 1e3, 3),
                 "alpha_best": float(g_res["alpha_best"]), "roofline": g_roof,
                 "kernels": g_kern,
                 "note": "same candidates through G = X^T X: e.G.e^T per row from the "
                         "diagonal 256-tiles of G and twice the tiles above them, in bf16 "
                         "hi + lo halves (4*sum_tm rows_tm*(K-256*tm) flops, about 2.1*K^2 "
                         "at K=4096), plus G's upper tiles once per step (gram_build), "
                         "shared by the scale and clip searches"}
    stats_ms, stats_n = prof["stats"]
    stats_gbs = (T * K * X.itemsize) / (stats_ms / 1e3 / max(stats_n, 1)) / 1e9 if stats_n else None
    pack_ms, pack_n = prof["pack"]
    pack_bytes = (N * K * X.itemsize + N * K * cfg.bits / 8
                  + (N * K / cfg.group) * (2 + cfg.bits / 8) + K * 4) / len(Ws)
    pack_gbs = pack_bytes / (pack_ms / 1e3 / max(pack_n, 1)) / 1e9 if pack_n else None

    out = {
        "metric": "AWQ alpha-candidates evaluated/sec (4096x4096, 64K tok, g128) + MFMA util %",
        "value": round(value, 3),
        "all_candidates_per_s": round(cands_per_step * args.steps / elapsed, 3),
        "unit": "alpha-candidates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": name, "T": T, "N": N, "K": K, "group": cfg.group, "bits": cfg.bits,
                   "zero_point": zp, "n_alpha": cfg.n_alpha, "n_ratio": cfg.n_ratio,
                   "pack": cfg.pack, "layers": list(cfg.layers) or None, "method": method},
        "roofline": roofline,
        "mfma_util_pct": (None if roofline["mfma_util_counters"] is None
                          else round(100 * roofline["mfma_util_counters"]["frac"], 1)),
        "hbm": {"stats_GBps": None if stats_gbs is None else round(stats_gbs, 1),
                "pack_GBps": None if pack_gbs is None else round(pack_gbs, 1),
                "peak_GBps": HBM_PEAK_GBS,
                "timing": "HIP events around each launch; they include the launch's own "
                          "few microseconds, a large part of a 4096x4096 pack (about 11 us "
                          "of kernel time in a kernel trace)"},
        "kernels": kernels,
        "alpha_best": float(res["alpha_best"]),
        "mse_alpha0": float(res["mse"][0]),
        "mse_best": float(res["mse"].min()),
    }
    if other is not None:
        out["gram"] = other
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, X, Ws, alphas, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
