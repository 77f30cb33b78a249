"""GPU parity of the Gram-matrix searches (E·G·Eᵀ per candidate row), through the C ABI.

The Gram path sees the same bf16 candidate operands E as the direct path, so
the same float64 "model" (exact sums of the bf16 operands) is the target. Its
own float32 arithmetic, with u = 2^-23:
  * G = XᵀX summed over T tokens: |Ĝ - G| <= γ_T·|X|ᵀ|X| entrywise;
  * the split G_hi + G_lo differs from Ĝ by at most 2^-16·|Ĝ|;
  * Z = (G_hi + G_lo)·e sums 2K products: γ_2K·(|Ĝ||e|);
  * M = Σ_j Z_j·e_j sums at most K products: γ_K·Σ_j |Z_j||e_j|.
All of it is bounded by (γ_T + 2^-16 + γ_2K + γ_K)·1.01·S with
S = |e|ᵀ(|X|ᵀ|X|)|e| = Σ_t (Σ_k |x_tk||e_k|)², which the test computes per
row; γ_n = n·u / (1 - n·u). The curve is also held to 1e-3 of the float64
oracle and to the α rule against the oracle's curve, as for the direct path,
and the Gram path is compared with the direct path on the GPU. The Gram path
has no split-operand form, so its one-token layer (whose single bf16 operands
leave 1.4e-3 on the curve, nothing to average over) is held to the bounds
only (``curve_rule=False``).
"""
import numpy as np
import pytest
import torch

import oracle as O
from post_weight_quantization_26_amd import synth
from test_gpu_parity import (MSE_REL, TIE_REL, assert_curve_rules, bits32, row_references,
                             to_dev)

pytestmark = pytest.mark.gpu

U = 2.0 ** -23


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    from post_weight_quantization_26_amd import api as A
    return A


def gamma(n):
    return n * U / (1 - n * U)


def gram_bound(T, K, S):
    return (gamma(T) + 2.0 ** -16 + gamma(2 * K) + gamma(K)) * 1.01 * S


def check_gram_scale(api, X, W, alphas, bits, zp, rows=None, group=128, curve_rule=True):
    Xd, Wd = to_dev(X, "bf16"), to_dev(W, "bf16")
    abar = api.act_stats(Xd)
    res = api.search_scale(Xd, Wd, abar, alphas, bits=bits, group=group, zero_point=zp,
                           want_row_sums=True, method="gram")
    dref = api.search_scale(Xd, Wd, abar, alphas, bits=bits, group=group, zero_point=zp,
                            want_row_sums=True)
    ref = O.search_scale(X, W, "bf16", O.act_stats(X, "bf16"), alphas, bits, group, zp,
                         rows=rows)
    T, N = X.shape[0], W.shape[0]
    K = X.shape[1]
    rs = res["row_sums"].cpu().numpy()
    drs = dref["row_sums"].cpu().numpy()
    assert np.allclose(rs.sum(axis=1) / (T * N), res["mse"], rtol=1e-12, atol=0)
    assert np.array_equal(bits32(res["s_best"]), ref["s_table"][res["index"]].view(np.uint32))
    sel = slice(None) if rows is None else np.asarray(rows)
    w_rows = O.decode(W, "bf16")[sel]
    cands = [(ref["s_table"][i], 1.0, (bits, group, zp)) for i in range(len(alphas))]
    M64, Mm, tol, S = row_references(X, "bf16", w_rows, cands, want_S=True)
    bound = gram_bound(T, K, S)
    worst = (np.abs(rs[:, sel] - Mm) / bound).max()
    assert worst <= 1.0, f"Gram rows vs model exceed the bound ({worst:.2f}x)"
    # against the direct path: each within its own bound of the same model
    assert np.all(np.abs(rs[:, sel] - drs[:, sel]) <= bound + tol)
    rel_direct = (np.abs(rs - drs) / drs).max()
    if rows is None:
        # the curve: within the summed bounds of the model's curve, and the
        # rules against the float64 oracle
        m_curve = Mm.sum(axis=1) / (T * N)
        assert np.all(np.abs(res["mse"] - m_curve) <= bound.sum(axis=1) / (T * N))
        print(f"gram: |gpu-model|/bound {worst:.2e}; vs direct max rel {rel_direct:.2e}")
        assert_curve_rules(res["mse"], res["index"], ref["mse"], "gram curve", curve_rule)
    else:
        print(f"gram: |gpu-model|/bound {worst:.2e}; vs direct max rel {rel_direct:.2e}")
    # the two paths choose the same α unless their curves nearly tie there
    d_mse = dref["mse"]
    if res["index"] != dref["index"]:
        a, b = d_mse[res["index"]], d_mse[dref["index"]]
        assert abs(a - b) / min(a, b) < TIE_REL, (res["index"], dref["index"], d_mse)
    return res, dref, Xd, Wd


def g_prime_from_gs(Gs_bytes, K):
    """G' (G on diagonal 256-tiles, 2G above them; NaN below) decoded from
    the hi/lo layout: row j, column c of its row tile's part holds hi at
    256·(c // 128) + c % 128 and lo 128 further on."""
    gs = Gs_bytes.view(np.uint16).reshape(K, 2 * K + 256)
    f = lambda h: (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    c = np.arange(K)
    # tiles below the diagonal are never written and may hold signalling NaN
    # bit patterns, whose widening raises numpy's invalid-value warning
    with np.errstate(invalid="ignore"):
        hi = f(gs[:, 256 * (c // 128) + c % 128])
        lo = f(gs[:, 256 * (c // 128) + 128 + c % 128])
    G = hi + lo
    tile = np.arange(K) // 256
    G[tile[:, None] > tile[None, :]] = np.nan
    return G


@pytest.mark.parametrize("T,K", [(700, 384), (1000, 640), (65, 128), (4160, 1152), (1100, 4096)])
def test_gram_matrix_elementwise(api, T, K):
    """G from X in place (transposing LDS reads, token slices, the XCD order
    from 1024 units on: 1100 tokens at K = 4096 make 9 slices x 136 tiles)
    against the float64 G of the oracle, every stored entry: within
    γ_T·(|X|ᵀ|X|) for the float32 sums plus 2^-16 for the hi/lo split,
    doubled above the diagonal tiles. Ragged T and a 128-channel last tile
    included."""
    X, _ = synth.make_custom(T, 8, K, "bf16", seed=300 + T + K)
    G = api.gram_build(to_dev(X, "bf16"))
    torch.cuda.synchronize()
    Gd = g_prime_from_gs(G.cpu().numpy(), K)
    G64 = O.gram_matrix(X, "bf16")
    xa = np.abs(O.decode(X, "bf16").astype(np.float64))
    A = xa.T @ xa
    tile = np.arange(K) // 256
    w = np.where(tile[:, None] < tile[None, :], 2.0, 1.0)
    upper = tile[:, None] <= tile[None, :]
    ref = w * G64
    bound = w * (gamma(T) * A + 2.0 ** -16 * np.abs(G64)) * 1.01
    err = np.abs(Gd - ref)
    worst = (err[upper] / np.maximum(bound[upper], 1e-300)).max()
    print(f"G {T}x{K}: max |err|/bound {worst:.2e}")
    assert np.all(np.isfinite(Gd[upper]))
    assert worst <= 1.0


@pytest.mark.parametrize("bits,zp", [(4, True), (3, True), (4, False)])
def test_gram_scale_small_ragged(api, bits, zp):
    # 700 tokens (padded to 768), 384 channels (two 256-row tiles of G, one
    # ragged), 300 rows per candidate
    X, W = synth.make_custom(700, 300, 384, "bf16", seed=140)
    check_gram_scale(api, X, W, synth.alpha_grid(7), bits, zp)


def test_gram_scale_one_token_and_group32(api):
    # one token: held to the bounds, not to the curve rules (module docstring)
    X, W = synth.make_custom(1, 40, 256, "bf16", n_out=2, seed=141)
    check_gram_scale(api, X, W, synth.alpha_grid(5), 4, True, group=32, curve_rule=False)


def test_gram_scale_tile_aligned(api):
    X, W = synth.make_custom(2048, 512, 512, "bf16", seed=142)
    check_gram_scale(api, X, W, synth.alpha_grid(9), 4, True)


def test_gram_clip(api):
    X, W = synth.make_custom(900, 264, 384, "bf16", seed=143)
    Xd, Wd = to_dev(X, "bf16"), to_dev(W, "bf16")
    ab = O.act_stats(X, "bf16")
    s = O.scale_for_alpha(ab, 0.5)
    sd = torch.from_numpy(s).to("cuda:0")
    ratios = synth.ratio_grid(8)
    g = api.search_clip(Xd, Wd, sd, ratios, want_row_sums=True, method="gram")
    d = api.search_clip(Xd, Wd, sd, ratios, want_row_sums=True)
    ref = O.search_clip(X, W, "bf16", s, ratios)
    w32 = O.decode(W, "bf16")
    cands = [(s, np.full(264, r, np.float32), (4, 128, True)) for r in ratios]
    M64, Mm, tol, S = row_references(X, "bf16", w32, cands, want_S=True)
    rs = g["row_sums"].cpu().numpy()
    bound = gram_bound(900, 384, S)
    assert np.all(np.abs(rs - Mm) <= bound)
    gi = np.searchsorted(np.asarray(ratios), g["ratio_best"].cpu().numpy())
    cols = np.arange(264)
    assert np.all(Mm[gi, cols] <= Mm.min(axis=0) + bound[gi, cols] + bound[Mm.argmin(axis=0), cols])
    same = np.mean(g["ratio_best"].cpu().numpy() == d["ratio_best"].cpu().numpy())
    print(f"gram clip: {same:.1%} of rows pick the direct path's ratio; "
          f"{np.mean(gi == ref['index']):.1%} the oracle's")
    assert abs(g["mse_clip"] - ref["mse_clip"]) / ref["mse_clip"] <= MSE_REL


def test_gram_bench_layer_full(api):
    """The 4096x4096, 65,536-token layer: every row against the direct path,
    16 sampled rows against the float64 oracle and its model."""
    cfg = synth.CONFIGS["llama7b_attn_4096"]
    X, W = synth.make_layer(cfg)
    rows = np.unique(np.linspace(0, cfg.N - 1, 16).round().astype(np.int64))
    res, dref, Xd, Wd = check_gram_scale(api, X, W, synth.alpha_grid(cfg.n_alpha), cfg.bits,
                                         cfg.zero_point, rows=rows)
    rs = res["row_sums"].cpu().numpy()
    drs = dref["row_sums"].cpu().numpy()
    rel = np.abs(rs - drs) / drs
    print(f"gram vs direct, all {rs.size} rows: max rel {rel.max():.2e}, "
          f"curve max rel {(np.abs(res['mse'] - dref['mse']) / dref['mse']).max():.2e}")
    assert rel.max() <= 1e-3
    assert (np.abs(res["mse"] - dref["mse"]) / dref["mse"]).max() <= 1e-4
    del Xd, Wd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,N,K", [(700, 300, 384), (2048, 512, 1024)])
def test_prepared_g_equals_built_in(api, T, N, K):
    """One G from gram_build serves the scale, clip and group searches; each
    equals, bit for bit, the search that builds G in its own workspace."""
    X, W = synth.make_custom(T, N, K, "bf16", seed=150 + K)
    W2 = synth.make_weight(136, K, 0.02, "bf16", seed=151 + K)
    Xd, Wd, W2d = to_dev(X, "bf16"), to_dev(W, "bf16"), to_dev(W2, "bf16")
    abar = api.act_stats(Xd)
    alphas = synth.alpha_grid(5)
    G = api.gram_build(Xd)
    assert G.numel() == api.gram_bytes(K)
    a = api.search_scale(Xd, Wd, abar, alphas, want_row_sums=True, method="gram")
    b = api.search_scale(Xd, Wd, abar, alphas, want_row_sums=True, method="gram", G=G)
    assert np.array_equal(a["mse"], b["mse"]) and a["index"] == b["index"]
    assert torch.equal(a["row_sums"], b["row_sums"]) and torch.equal(a["s_best"], b["s_best"])
    ratios = synth.ratio_grid(6)
    c = api.search_clip(Xd, Wd, a["s_best"], ratios, want_row_sums=True, method="gram")
    d = api.search_clip(Xd, Wd, a["s_best"], ratios, want_row_sums=True, method="gram", G=G)
    assert c["mse_clip"] == d["mse_clip"]
    assert torch.equal(c["ratio_best"], d["ratio_best"]) and torch.equal(c["row_sums"], d["row_sums"])
    e = api.search_scale_group(Xd, [Wd, W2d], abar, alphas, want_row_sums=True, method="gram")
    f = api.search_scale_group(Xd, [Wd, W2d], abar, alphas, want_row_sums=True, method="gram",
                               G=G)
    assert np.array_equal(e["mse"], f["mse"]) and torch.equal(e["row_sums"], f["row_sums"])
    # G is only read: a second use gives the same again
    g = api.search_scale(Xd, Wd, abar, alphas, method="gram", G=G)
    assert np.array_equal(g["mse"], b["mse"])


def test_prepared_g_bench_layer(api):
    """The 4096x4096, 65,536-token layer: scale and clip searches through one
    prepared G equal the building searches bit for bit."""
    cfg = synth.CONFIGS["llama7b_attn_4096"]
    X, W = synth.make_layer(cfg)
    Xd, Wd = to_dev(X, "bf16"), to_dev(W, "bf16")
    abar = api.act_stats(Xd)
    alphas = synth.alpha_grid(cfg.n_alpha)
    G = api.gram_build(Xd)
    a = api.search_scale(Xd, Wd, abar, alphas, method="gram")
    b = api.search_scale(Xd, Wd, abar, alphas, method="gram", G=G)
    assert np.array_equal(a["mse"], b["mse"]) and torch.equal(a["s_best"], b["s_best"])
    ratios = synth.ratio_grid(10)
    c = api.search_clip(Xd, Wd, a["s_best"], ratios, method="gram")
    d = api.search_clip(Xd, Wd, a["s_best"], ratios, method="gram", G=G)
    assert c["mse_clip"] == d["mse_clip"] and torch.equal(c["ratio_best"], d["ratio_best"])
    del Xd, Wd, G
    torch.cuda.empty_cache()
