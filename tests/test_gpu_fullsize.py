"""GPU parity at the full Llama-class layer sizes, whole layers against the oracle.

Each workload runs at its full size, in the launch configuration the
benchmark times, and is checked three ways:

  * Whole layer against the float64 oracle (``tests/fullsize_oracle.py``: the
    oracle's Gram route by row blocks, computed in the test, or for the
    70B-class layer read from ``tests/golden/oracle_llama70b_mlp.json``, which
    ``tests/golden/make_oracle_fullsize.py`` wrote from the oracle alone):
    every α's MSE within 1e-3 relative; the chosen α identical unless the
    oracle's two best are within 1e-4; with s at the oracle's best α, every
    clip ratio's MSE Σ_n M_n(r) / (T·N) and mse_clip within 1e-3; per output
    row, the chosen ratio identical unless the oracle's two best for that row
    are within 1e-4 (rows that break it are counted and reported; with split
    candidate operands none may).
  * 16 evenly spaced rows against the oracle's direct route and the model of
    the bf16 operands, per row within the float32 bound (as in
    ``test_gpu_parity``).
  * The packed layer, with the oracle's s* and r*, bit for bit against the
    oracle over the whole layer.
"""
import numpy as np
import pytest
import torch

import fullsize_oracle as F
import oracle as O
from post_weight_quantization_26_amd import synth
from test_gpu_parity import (assert_curve_rules, assert_pack_parity, check_clip,
                             check_scale_search, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    from post_weight_quantization_26_amd import api as A
    return A


def sample_rows(N, k=16):
    return np.unique(np.linspace(0, N - 1, k).round().astype(np.int64))


def log(msg):
    print(msg, flush=True)


def check_clip_full(api, Xd, Wd, cfg, zp, s_best, full, split_e):
    """Whole-layer clip search at the oracle's s* against the oracle's results."""
    ratios = np.asarray(full["ratios"], np.float32)
    res = api.search_clip(Xd, Wd, torch.from_numpy(s_best).to("cuda:0"), ratios, bits=cfg.bits,
                          group=cfg.group, zero_point=zp, want_row_sums=True, split_e=split_e)
    rs = res["row_sums"].cpu().numpy()
    curve = rs.sum(axis=1) / (cfg.T * cfg.N)
    ref_curve = np.asarray(full["clip_curve"])
    crel = (np.abs(curve - ref_curve) / ref_curve).max()
    rel = abs(res["mse_clip"] - full["mse_clip"]) / full["mse_clip"]
    gi = np.searchsorted(ratios, res["ratio_best"].cpu().numpy())
    best = F.from_letters(full["row_best"])
    decided = F.from_letters(full["row_near_tie"]) == ord("0") - 65
    bad = int(np.sum(decided & (gi != best)))
    log(f"{cfg.name} zp={zp} split={split_e}: ratio curve max rel err {crel:.2e}, mse_clip rel "
        f"err {rel:.2e}; {np.mean(gi == best):.2%} of rows pick the oracle's ratio, {bad} of "
        f"{cfg.N} break the per-row rule ({int(np.sum(~decided))} oracle near-ties)")
    assert crel <= 1e-3 and rel <= 1e-3
    if split_e:
        assert bad == 0, f"{bad} rows pick a ratio the oracle rules out"
    return ratios[best]


_CACHE = {}


def layer_and_oracle(name):
    """Inputs and the oracle's whole-layer results of one workload; the last
    workload's are kept for the next test (the split and single-operand runs
    of a workload share them)."""
    if name not in _CACHE:
        _CACHE.clear()
        cfg = synth.CONFIGS[name]
        X, W = synth.make_layer(cfg)
        _CACHE[name] = (X, W, F.stored_or_live(name, X, W, log=log))
    return _CACHE[name]


def run_config(api, name, split_e=False, variants=None):
    cfg = synth.CONFIGS[name]
    X, W, full = layer_and_oracle(name)
    rows = sample_rows(cfg.N)
    alphas = synth.alpha_grid(cfg.n_alpha)
    ref_abar = O.act_stats(X, cfg.dtype)
    s_table = O.scale_table(ref_abar, alphas)
    for zp in (variants or cfg.variants):
        v = full["variants"]["asym" if zp else "sym"]
        res, _, Xd, Wd = check_scale_search(api, X, W, cfg.dtype, alphas, cfg.bits, zp,
                                            rows=rows, group=cfg.group, split_e=split_e)
        log(f"{name} zp={zp} split={split_e}: alpha* {res['alpha_best']:.4f} "
            f"(oracle {v['alpha_best']:.4f})")
        assert_curve_rules(res["mse"], res["index"], np.asarray(v["mse"]),
                           f"{name} zp={zp} split={split_e} alpha curve")
        # the clip search and the pack take the oracle's s*, so a near-tie
        # flip of α cannot cascade into them
        s_best = s_table[v["index"]]
        ratio = None
        if cfg.n_ratio:
            check_clip(api, Xd, Wd, X, W, cfg.dtype, s_best, np.asarray(v["ratios"], np.float32),
                       cfg.bits, zp, rows=rows, group=cfg.group, split_e=split_e)
            ratio = check_clip_full(api, Xd, Wd, cfg, zp, s_best, v, split_e)
        if cfg.pack and not split_e:
            qw, qz, sc = api.quantize_pack(Wd, torch.from_numpy(s_best).to("cuda:0"),
                                           None if ratio is None else
                                           torch.from_numpy(ratio).to("cuda:0"),
                                           bits=cfg.bits, group=cfg.group, zero_point=zp)
            assert_pack_parity(qw, qz, sc, W, cfg.dtype, s_best, ratio, zp, cfg.bits, cfg.group)
        del Xd, Wd
        torch.cuda.empty_cache()


@pytest.mark.parametrize("split_e", [False, True])
def test_llama7b_attn_4096_full(api, split_e):
    # the benchmark's layer: 4096 x 4096, 65,536 tokens, 20 alphas, pack
    run_config(api, "llama7b_attn_4096", split_e)


def test_llama7b_attn_4096_f16_full(api):
    # the same layer held in fp16: fp16 candidates on the fp16 MFMA, fp16 pack
    run_config(api, "llama7b_attn_4096_f16")


@pytest.mark.parametrize("split_e", [False, True])
def test_llama7b_mlp_up_full(api, split_e):
    # 11008 x 4096, 20 alphas then 20 clip ratios per output channel, then pack
    run_config(api, "llama7b_mlp_up", split_e)


@pytest.mark.parametrize("split_e", [False, True])
def test_llama7b_mlp_down_int3_full(api, split_e):
    # 4096 x 11008, heavy-tailed inputs, INT3 search, clip and 3-bit pack
    run_config(api, "llama7b_mlp_down_int3", split_e)


def test_llama7b_attn_4096_g32_full(api):
    # the benchmark's layer at group size 32: search and pack
    run_config(api, "llama7b_attn_4096_g32")


@pytest.mark.parametrize("split_e", [False, True])
def test_llama70b_mlp_full(api, split_e):
    # 28672 x 8192 over 32768 tokens, asymmetric and symmetric INT4, search +
    # clip + pack; the oracle's whole-layer results are stored
    run_config(api, "llama70b_mlp", split_e)
