"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerances:
  * ā, the scale table, zeros and fp16 scales: bit-exact. Codes: bit-exact
    except elements whose pre-round value fl32(w'/step) lies within 1e-6 of a
    .5 boundary (the kernels form the quotient from the group's reciprocal
    with one FMA correction, at most one ulp from IEEE division); such
    elements are counted and may differ by one code.
  * Per-candidate MSE (the curve) against the float64 oracle: 1e-3 relative.
  * Chosen α: identical unless the oracle's two best MSEs are within 1e-4
    relative.
  * Per-row clip ratio r*_n: the same rule per row (identical unless the
    oracle's two best errors of that row are within 1e-4 relative). Rows
    that break it are counted and reported; with split candidate operands
    (split_e) none may.
  * Per-row output errors M_n: the search GEMM consumes the candidates' error
    weights E = Ŵ - W as bf16 MFMA operands. The test rebuilds exactly those
    operands from the oracle's codes (the kernel's float32 arithmetic, then
    one bf16 rounding) and computes their M_n in float64 ("model"). GPU and
    model may then differ only by float32 accumulation inside the MFMA and in
    the per-tile sums of squares; the test computes that worst-case bound per
    row (γ_K = K·2^-23 / (1 - K·2^-23) on Σ_j |x_tj e_nj|, plus 300·2^-23 for
    the sums of squares) and requires |GPU - model| within it. The gap between
    the model and the float64 oracle is the cost of bf16 operands; it is
    reported. With split_e the operands are hi + lo halves (the model
    rebuilds them the same way) and the bound covers 2K products per output.
  * Clip ratio per row: the GPU's pick is optimal for the model up to the
    model tolerance, and its float64 regret is within the row's bf16 gap.

The curve rule and the α rule are asserted exactly as stated above for every
layer, with one documented exception: a layer whose error is carried by a few
rows or tokens (one row of much larger weights; one token) does not average
out the rounding of single 16-bit candidate operands, which leaves up to ~2e-3
on its curve. Those layers are held to the rules with split_e, and with
single operands to the per-row float32 bound against the model only
(``curve_rule=False``, used by the tests that say so).
"""
import numpy as np
import pytest
import torch

import oracle as O
from post_weight_quantization_26_amd import synth

pytestmark = pytest.mark.gpu

MSE_REL = 1e-3
TIE_REL = 1e-4
U_F32 = 2.0 ** -23     # covers round-to-nearest and truncating float32 accumulation


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    from post_weight_quantization_26_amd import api as A
    return A


def to_dev(a, dtype):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.float16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda:0")


def bits32(t):
    return t.detach().cpu().numpy().view(np.uint32)


def assert_alpha_rule(gpu_idx, ref_mse):
    order = np.argsort(ref_mse, kind="stable")
    best, second = ref_mse[order[0]], ref_mse[order[1]] if len(order) > 1 else np.inf
    if (second - best) / best >= TIE_REL:
        assert gpu_idx == order[0], (gpu_idx, order[:2], ref_mse)
    else:
        assert gpu_idx in order[:2]


def _round16(e, dtype):
    """float32 -> the MFMA operand type (RNE), back as float32."""
    if dtype == "f16":
        return e.astype(np.float16).astype(np.float32)
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(e))


def model_E(w32, s32, ratio, bits, zp, dtype, group=128, split=False, magnitude=False):
    """Error weights as the search GEMM consumes them, from the oracle's codes
    and the kernel's float32 arithmetic: fl32(fl32(fl32((q - zero)·step) ·
    fl32(1/s)) - w), then one RNE rounding to the MFMA operand type (bf16 or
    fp16; float32 inputs stay float32). split: hi = rnd(e), lo = rnd(e - hi)
    and the operand is hi + lo (magnitude: |hi| + |lo|, for the bound)."""
    q, step, zero = O.quantize(w32, s32, ratio, bits, group, zp)
    N, K = w32.shape
    d = ((q.reshape(N, K // group, group).astype(np.float32) - zero[:, :, None]) * step[:, :, None])
    inv_s = (np.float32(1.0) / s32.astype(np.float32)).astype(np.float32)
    e = (d.reshape(N, K) * inv_s[None, :]) - w32
    e = e.astype(np.float32)
    if dtype == "f32":
        return np.abs(e).astype(np.float64) if magnitude else e.astype(np.float64)
    hi = _round16(e, dtype)
    if not split:
        return np.abs(hi).astype(np.float64) if magnitude else hi.astype(np.float64)
    lo = _round16((e - hi).astype(np.float32), dtype)
    if magnitude:
        return np.abs(hi).astype(np.float64) + np.abs(lo).astype(np.float64)
    return hi.astype(np.float64) + lo.astype(np.float64)


def row_references(X, dtype, w_rows, cands, chunk=4096, want_S=False, split=False):
    """One pass over X for stacked candidates [(s, ratio), ...] on rows w_rows.

    Returns M64 (float64 oracle errors), Mm (model errors) and tol (worst-case
    float32 accumulation bound of the direct GEMM), each [n_cand, R]; with
    want_S also S = Σ_t (Σ_k |x_tk|·|e_k|)² per row (= |e|ᵀ(|X|ᵀ|X|)|e|).
    split: the model's operands are hi + lo halves; the GEMM sums 2K products."""
    e64 = np.concatenate([O.candidate_weights(w_rows, s, r, *c) - w_rows.astype(np.float64)
                          for (s, r, c) in cands])
    em = np.concatenate([model_E(w_rows, s, r, c[0], c[2], dtype, c[1], split)
                         for (s, r, c) in cands])
    Rt, K = e64.shape
    M64, Mm, acc, acc2 = (np.zeros(Rt) for _ in range(4))
    aem = np.concatenate([model_E(w_rows, s, r, c[0], c[2], dtype, c[1], split, magnitude=True)
                          for (s, r, c) in cands]).T
    for t0 in range(0, X.shape[0], chunk):
        x = O.decode(X[t0:t0 + chunk], dtype).astype(np.float64)
        y = x @ e64.T
        ym = x @ em.T
        a = np.abs(x) @ aem
        M64 += (y * y).sum(axis=0)
        Mm += (ym * ym).sum(axis=0)
        acc += (np.abs(ym) * a).sum(axis=0)
        acc2 += (a * a).sum(axis=0)
    Ke = 2 * K if split and dtype != "f32" else K
    g = Ke * U_F32 / (1 - Ke * U_F32)
    tol = 2 * g * acc + g * g * acc2 + 300 * U_F32 * Mm
    n = len(cands)
    if want_S:
        return M64.reshape(n, -1), Mm.reshape(n, -1), tol.reshape(n, -1), acc2.reshape(n, -1)
    return M64.reshape(n, -1), Mm.reshape(n, -1), tol.reshape(n, -1)


def _ratio(num, den):
    """max of num/den over den > 0 (0 when there is none)."""
    pos = den > 0
    return float((num[pos] / den[pos]).max()) if pos.any() else 0.0


def compare_rows(gpu_rows, M64, Mm, tol, what):
    err = np.abs(gpu_rows - Mm)
    # a row whose candidate error is exactly zero (an all-zero weight row
    # quantises exactly) has a zero bound and must come out exactly zero
    assert np.all(err[tol == 0] == 0), f"{what}: a zero-error row is not zero on the GPU"
    worst = _ratio(err, tol)
    assert worst <= 1.0, f"{what}: GPU vs model exceeds the float32 bound ({worst:.2f}x)"
    gap = _ratio(np.abs(Mm - M64), M64)
    print(f"{what}: |gpu-model|/bound max {worst:.2e}; 16-bit operand gap max {gap:.2e}; "
          f"|gpu-oracle|/oracle max {_ratio(np.abs(gpu_rows - M64), M64):.2e}")


def check_scale_search(api, X, W, dtype, alphas, bits, zp, rows=None, ws=None, group=128,
                       split_e=False, curve_rule=True):
    """Runs stats + search on the GPU and the oracle; compares. Returns both results.
    curve_rule=False (only for the layers the module docstring names) keeps
    every check except the curve and α rules against the float64 oracle."""
    Xd, Wd = to_dev(X, dtype), to_dev(W, dtype)
    abar = api.act_stats(Xd)
    ref_abar = O.act_stats(X, dtype)
    assert np.array_equal(bits32(abar), ref_abar.view(np.uint32)), "abar differs"
    res = api.search_scale(Xd, Wd, abar, alphas, bits=bits, group=group, zero_point=zp,
                           want_row_sums=True, ws=ws, split_e=split_e)
    ref = O.search_scale(X, W, dtype, ref_abar, alphas, bits, group, zp, rows=rows)
    T, N = X.shape[0], W.shape[0]
    rs = res["row_sums"].cpu().numpy()
    # the curve is the mean of the per-row sums (any size)
    assert np.allclose(rs.sum(axis=1) / (T * N), res["mse"], rtol=1e-12, atol=0)
    # s_best is the scale row of the chosen α, bit for bit
    assert np.array_equal(bits32(res["s_best"]), ref["s_table"][res["index"]].view(np.uint32))
    sel = slice(None) if rows is None else np.asarray(rows)
    w_rows = O.decode(W, dtype)[sel]
    cands = [(ref["s_table"][i], 1.0, (bits, group, zp)) for i in range(len(alphas))]
    M64, Mm, tol = row_references(X, dtype, w_rows, cands, split=split_e)
    assert np.allclose(M64, ref["row_sums"], rtol=1e-10, atol=0)
    compare_rows(rs[:, sel], M64, Mm, tol, "alpha search rows")
    if rows is None:
        # the curve against the model, within the summed float32 bounds (any size)
        assert np.all(np.abs(res["mse"] - Mm.sum(axis=1) / (T * N)) <= tol.sum(axis=1) / (T * N))
        assert_curve_rules(res["mse"], res["index"], ref["mse"], "alpha curve", curve_rule)
    return res, ref, Xd, Wd


def assert_curve_rules(gpu_mse, gpu_idx, ref_mse, what, curve_rule=True):
    """Per-candidate MSE within 1e-3 relative of the float64 oracle, and the
    oracle's argmin unless its two best values are within 1e-4 relative."""
    mrel = np.abs(np.asarray(gpu_mse) - ref_mse) / ref_mse
    print(f"{what}: max rel err vs oracle {mrel.max():.2e}"
          + ("" if curve_rule else " (rules not asserted: single operands, few rows)"))
    if curve_rule:
        assert mrel.max() <= MSE_REL, f"{what}: mse rel err {mrel.max():.3e}"
        assert_alpha_rule(gpu_idx, ref_mse)


def clip_row_rule(gpu_idx, ref_rows):
    """Rows whose GPU ratio index breaks the α rule applied per row: it differs
    from the oracle's argmin although the oracle's two best errors of the row
    are 1e-4 or more apart (relative). Returns their count."""
    order = np.argsort(ref_rows, axis=0, kind="stable")
    cols = np.arange(ref_rows.shape[1])
    best, second = ref_rows[order[0], cols], ref_rows[order[1], cols]
    with np.errstate(divide="ignore", invalid="ignore"):
        decided = np.where(best > 0, (second - best) / best, np.inf) >= TIE_REL
    return int(np.sum(decided & (gpu_idx != order[0])))


def check_clip(api, Xd, Wd, X, W, dtype, s, ratios, bits, zp, rows=None, group=128,
               split_e=False, curve_rule=True):
    T, N = X.shape[0], W.shape[0]
    ratios = np.asarray(ratios, np.float32)
    res = api.search_clip(Xd, Wd, torch.from_numpy(s).to("cuda:0"), ratios, bits=bits,
                          group=group, zero_point=zp, want_row_sums=True, split_e=split_e)
    ref = O.search_clip(X, W, dtype, s, ratios, bits, group, zp, rows=rows)
    rs = res["row_sums"].cpu().numpy()
    sel = slice(None) if rows is None else np.asarray(rows)
    w_rows = O.decode(W, dtype)[sel]
    R = w_rows.shape[0]
    cands = [(s, np.full(R, r, np.float32), (bits, group, zp)) for r in ratios]
    M64, Mm, tol = row_references(X, dtype, w_rows, cands, split=split_e)
    assert np.allclose(M64, ref["row_sums"], rtol=1e-10, atol=0)
    compare_rows(rs[:, sel], M64, Mm, tol, "clip search rows")
    rb = res["ratio_best"].cpu().numpy()
    assert np.all(np.isin(rb, ratios))
    gi = np.searchsorted(ratios, rb[sel])
    cols = np.arange(R)
    # optimal for the model up to the model tolerance
    assert np.all(Mm[gi, cols] <= Mm.min(axis=0) + tol[gi, cols] + tol[Mm.argmin(axis=0), cols])
    # float64 regret within the row's bf16 gap (both candidates' gaps)
    gap = np.abs(Mm - M64)
    assert np.all(M64[gi, cols] - M64.min(axis=0) <=
                  gap[gi, cols] + gap[ref["index"], cols] + tol[gi, cols] + tol[ref["index"], cols])
    bad = clip_row_rule(gi, M64)
    print(f"clip: {np.mean(gi == ref['index']):.1%} of rows pick the oracle's ratio; "
          f"{bad} of {R} rows break the per-row rule")
    if split_e:
        assert bad == 0, f"{bad} rows pick a ratio the oracle rules out"
    best = rs.min(axis=0)
    assert np.isclose(res["mse_clip"], best.sum() / (T * N), rtol=1e-12)
    if rows is None:
        # the per-ratio curve and mse_clip against the float64 oracle
        ratio_curve = rs.sum(axis=1) / (T * N)
        ref_curve = ref["row_sums"].sum(axis=1) / (T * N)
        rel = abs(res["mse_clip"] - ref["mse_clip"]) / ref["mse_clip"]
        crel = (np.abs(ratio_curve - ref_curve) / ref_curve).max()
        print(f"clip: mse_clip rel err {rel:.2e}, ratio curve max rel err {crel:.2e}")
        if curve_rule:
            assert rel <= MSE_REL and crel <= MSE_REL
    return res, ref


# ---------------------------------------------------------------------------
# step 1 and 2
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("T,K", [(1, 8), (7, 264), (300, 1000), (5000, 4096)])
def test_act_stats_bitwise(api, dtype, T, K):
    if dtype == "f32":
        K = K - K % 4
    if dtype == "f16":
        x = np.random.default_rng(T + K).standard_normal((T, K)).astype(np.float32) * 3
        X = x.astype(np.float16).view(np.uint16)
    else:
        X = synth.make_activations(T, K, max(1, K // 100), 20.0, 100.0, dtype, seed=T * 7 + K)
    got = api.act_stats(to_dev(X, dtype))
    ref = O.act_stats(X, dtype)
    assert np.array_equal(bits32(got), ref.view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_act_stats_one_batch_equals_single_call(api, dtype):
    """One batch through accumulate + finalize is the single call, bit for bit
    (same partials, same fixed-order sum, added to zero, same division)."""
    x = np.random.default_rng(11).standard_normal((3000, 1000)).astype(np.float32) * 4
    X = {"bf16": synth.f32_to_bf16_bits(x), "f16": x.astype(np.float16).view(np.uint16),
         "f32": x}[dtype]
    Xd = to_dev(X, dtype)
    sums = torch.zeros(1000, dtype=torch.float64, device="cuda:0")
    api.act_stats_accumulate(Xd, sums)
    got = api.act_stats_finalize(sums, 3000)
    assert np.array_equal(bits32(got), bits32(api.act_stats(Xd)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_act_stats_batches(api, dtype):
    """Calibration batches of uneven length (one of a single token): the mean
    over all their tokens, as the oracle computes it on the concatenation."""
    K = 4096 if dtype == "bf16" else 1000
    sizes = (300, 1, 5000, 77)
    batches = [synth.make_activations(T, K, K // 100, 20.0, 100.0, dtype, seed=40 + i)
               for i, T in enumerate(sizes)]
    sums = torch.zeros(K, dtype=torch.float64, device="cuda:0")
    for Xb in batches:
        api.act_stats_accumulate(to_dev(Xb, dtype), sums)
    got = api.act_stats_finalize(sums, sum(sizes))
    ref = O.act_stats(np.concatenate(batches), dtype)
    assert np.array_equal(bits32(got), ref.view(np.uint32))


def test_scale_table_bitwise(api):
    X = synth.make_activations(2048, 4096, 41, 20.0, 100.0, "bf16", seed=3)
    ab = O.act_stats(X, "bf16")
    alphas = synth.alpha_grid(20)
    got = api.scale_table(torch.from_numpy(ab).to("cuda:0"), alphas)
    ref = O.scale_table(ab, alphas)
    d = np.abs(bits32(got).astype(np.int64) - ref.view(np.uint32).astype(np.int64))
    assert d.max() <= 1, "scale table differs by more than one ulp"
    assert (d > 0).sum() <= 2, f"{(d > 0).sum()} scale values differ"
    assert np.array_equal(bits32(got)[0], np.ones(4096, np.float32).view(np.uint32))


# ---------------------------------------------------------------------------
# steps 3-6: the α search
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits,zp", [(4, True), (3, True), (4, False)])
def test_search_scale_small_ragged(api, bits, zp):
    # 3 token tiles (last ragged), 2 candidate tiles per α with a ragged tail, 3 groups
    X, W = synth.make_custom(700, 300, 384, "bf16", seed=21)
    check_scale_search(api, X, W, "bf16", synth.alpha_grid(7), bits, zp)


def test_search_scale_tile_aligned(api):
    X, W = synth.make_custom(512, 256, 256, "bf16", seed=22)
    check_scale_search(api, X, W, "bf16", synth.alpha_grid(5), 4, True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("bits,zp,group", [(4, True, 128), (3, True, 64), (4, False, 32)])
def test_search_split_small_ragged(api, dtype, bits, zp, group):
    """Split candidate operands (hi + lo halves, the main loop's pair mode):
    the model bound over 2K products per row, the curve rules, and the
    per-row clip rule with no exception allowed."""
    X, W = synth.make_custom(700, 300, 384, dtype, seed=91 + bits + group)
    res, ref, Xd, Wd = check_scale_search(api, X, W, dtype, synth.alpha_grid(7), bits, zp,
                                          group=group, split_e=True)
    check_clip(api, Xd, Wd, X, W, dtype, ref["s_table"][res["index"]], synth.ratio_grid(6),
               bits, zp, group=group, split_e=True)


def test_search_split_group_and_batches(api):
    """A split group search equals the split search of the stacked weights,
    and a workspace for one candidate at a time gives the same bits."""
    X, _ = synth.make_custom(600, 8, 256, "bf16", seed=93)
    Ws = [synth.make_weight(n, 256, 0.02, "bf16", seed=94 + n) for n in (264, 40)]
    Xd = to_dev(X, "bf16")
    abar = api.act_stats(Xd)
    alphas = synth.alpha_grid(5)
    grp = api.search_scale_group(Xd, [to_dev(w, "bf16") for w in Ws], abar, alphas,
                                 want_row_sums=True, split_e=True)
    Wd = to_dev(np.concatenate(Ws), "bf16")
    stacked = api.search_scale(Xd, Wd, abar, alphas, want_row_sums=True, split_e=True)
    assert np.array_equal(grp["mse"], stacked["mse"])
    from post_weight_quantization_26_amd import _lib
    one = api.workspace_bytes_batch(_lib.AWQ_OP_SEARCH_SCALE_SPLIT_E, 600, 304, 256, 5, 1,
                                    torch.bfloat16)
    small = torch.empty(one, dtype=torch.uint8, device="cuda:0")
    b = api.search_scale(Xd, Wd, abar, alphas, want_row_sums=True, split_e=True, ws=small)
    assert np.array_equal(b["mse"], stacked["mse"])
    assert torch.equal(b["row_sums"], stacked["row_sums"])
    ref = O.search_scale_group(X, Ws, "bf16", O.act_stats(X, "bf16"), alphas)
    assert_curve_rules(grp["mse"], grp["index"], ref["mse"], "split group curve")


@pytest.mark.parametrize("split_e", [True, False])
def test_search_scale_degenerate_shapes(api, split_e):
    # one token, one output row, one group, a single α = 0 (plain rounding);
    # one row of one token: the curve rules hold with split operands
    X, W = synth.make_custom(1, 1, 128, "bf16", n_out=1, seed=23)
    res, ref, _, _ = check_scale_search(api, X, W, "bf16", np.array([0.0], np.float32), 4, True,
                                        split_e=split_e, curve_rule=split_e)
    assert res["alpha_best"] == 0.0
    assert np.array_equal(bits32(res["s_best"]), np.ones(128, np.float32).view(np.uint32))


def degenerate_layer(seed=26):
    """A 300-token, 288 x 512 layer whose values hit the quantiser's and the
    scale's floors: an all-zero weight row, a row whose second group is zero,
    a constant group, a group with a single nonzero, groups far below the
    1e-5 step floor, a large-magnitude row, and an all-zero activation
    column (its ā is 0 and is floored at 1e-8 in the scale)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((300, 512)).astype(np.float32)
    x[:, 7] = 0.0
    x[:, 100] *= 40.0                                  # an outlier channel
    w = (rng.standard_normal((288, 512)) * 0.02).astype(np.float32)
    w[3] = 0.0
    w[5, 128:256] = 0.0
    w[8, 0:128] = 0.0125
    w[9, 256:384] = 0.0
    w[9, 300] = -0.7
    w[11, :] = rng.standard_normal(512).astype(np.float32) * 1e-7
    w[12, 384:] = 3e-6
    w[13, :] *= 5000.0
    return synth.f32_to_bf16_bits(x), synth.f32_to_bf16_bits(w)


@pytest.mark.parametrize("split_e", [True, False])
@pytest.mark.parametrize("bits,zp", [(4, True), (3, True), (4, False)])
def test_degenerate_values_search_and_pack(api, bits, zp, split_e):
    """The layer's error is carried by one row of 5000x larger weights, so the
    rounding of single bf16 candidate operands does not average out over rows
    (1.9e-3 on its curve): the curve and α rules are asserted with split
    operands; single operands are held to the per-row float32 bound."""
    X, W = degenerate_layer()
    res, ref, Xd, Wd = check_scale_search(api, X, W, "bf16", synth.alpha_grid(7), bits, zp,
                                          split_e=split_e, curve_rule=split_e)
    s = ref["s_table"][res["index"]]
    check_clip(api, Xd, Wd, X, W, "bf16", s, synth.ratio_grid(6), bits, zp, split_e=split_e,
               curve_rule=split_e)
    qw, qz, sc = api.quantize_pack(Wd, torch.from_numpy(s).to("cuda:0"), bits=bits,
                                   zero_point=zp)
    assert_pack_parity(qw, qz, sc, W, "bf16", s, None, zp, bits=bits)


def test_non_finite_inputs_are_reported(api):
    """A NaN in X or an Inf in W makes the output error non-finite: the
    searches report AWQ_E_RANGE instead of an argmin over NaN, and the pack
    reports the non-finite fp16 scale the same way."""
    from post_weight_quantization_26_amd._lib import AwqError
    X, W = synth.make_custom(300, 264, 256, "bf16", seed=27)
    Xn = X.copy()
    Xn[5, 17] = 0x7FC0                                  # bf16 quiet NaN
    Xd, Wd = to_dev(Xn, "bf16"), to_dev(W, "bf16")
    abar = api.act_stats(Xd)
    for method in ("direct", "gram"):
        with pytest.raises(AwqError, match="not finite"):
            api.search_scale(Xd, Wd, abar, synth.alpha_grid(3), method=method)
    Wi = W.copy()
    Wi[2, 3] = 0x7F80                                   # bf16 +Inf
    Xd, Wd = to_dev(X, "bf16"), to_dev(Wi, "bf16")
    s = torch.ones(256, dtype=torch.float32, device="cuda:0")
    with pytest.raises(AwqError, match="not finite"):
        api.search_clip(Xd, Wd, s, synth.ratio_grid(3))
    with pytest.raises(AwqError, match="fp16"):
        api.quantize_pack(Wd, s)
    # the library stays usable afterwards
    Wd = to_dev(W, "bf16")
    res = api.search_scale(Xd, Wd, api.act_stats(Xd), synth.alpha_grid(3))
    assert np.all(np.isfinite(res["mse"]))


@pytest.mark.parametrize("bits,zp", [(4, True), (3, True), (4, False)])
def test_search_scale_f16(api, bits, zp):
    """fp16 layers (fp16 models): the candidates' error weights go to the
    GEMM as fp16; the model rounds them the same way."""
    X, W = synth.make_custom(700, 300, 384, "f16", seed=28)
    res, ref, Xd, Wd = check_scale_search(api, X, W, "f16", synth.alpha_grid(7), bits, zp)
    s = ref["s_table"][res["index"]]
    check_clip(api, Xd, Wd, X, W, "f16", s, synth.ratio_grid(6), bits, zp)


def test_search_scale_group_f16(api):
    X, _ = synth.make_custom(600, 8, 256, "f16", seed=29)
    Ws = [synth.make_weight(n, 256, 0.02, "f16", seed=30 + n) for n in (264, 40)]
    Xd = to_dev(X, "f16")
    abar = api.act_stats(Xd)
    alphas = synth.alpha_grid(5)
    grp = api.search_scale_group(Xd, [to_dev(w, "f16") for w in Ws], abar, alphas,
                                 want_row_sums=True)
    ref = O.search_scale_group(X, Ws, "f16", O.act_stats(X, "f16"), alphas, 4, 128, True)
    assert np.allclose(grp["mse"], ref["mse"], rtol=MSE_REL, atol=0)
    stacked = api.search_scale(Xd, to_dev(np.concatenate(Ws), "f16"), abar, alphas,
                               want_row_sums=True)
    assert np.array_equal(grp["mse"], stacked["mse"])


def test_search_scale_many_token_tiles(api):
    # 33 token tiles: exercises the XCD-grouped tile order with padding blocks
    X, W = synth.make_custom(33 * 256 - 5, 520, 256, "bf16", seed=24)
    check_scale_search(api, X, W, "bf16", synth.alpha_grid(3), 4, True)


@pytest.mark.parametrize("T", [4000, 2000, 1000])
def test_search_scale_4_8_16_token_tiles(api, T):
    # 16, 8 and 4 token tiles: the XCD-grouped order for few token tiles
    # (token groups x column groups), 7 column tiles with padding blocks
    X, W = synth.make_custom(T, 520, 256, "bf16", seed=T)
    check_scale_search(api, X, W, "bf16", synth.alpha_grid(3), 4, True)


def test_search_is_deterministic_and_batch_invariant(api):
    X, W = synth.make_custom(600, 264, 256, "bf16", seed=25)
    Xd, Wd = to_dev(X, "bf16"), to_dev(W, "bf16")
    abar = api.act_stats(Xd)
    alphas = synth.alpha_grid(6)
    a = api.search_scale(Xd, Wd, abar, alphas, want_row_sums=True)
    b = api.search_scale(Xd, Wd, abar, alphas, want_row_sums=True)
    from post_weight_quantization_26_amd import _lib
    need1 = api.workspace_bytes_batch(_lib.AWQ_OP_SEARCH_SCALE, 600, 264, 256, 6, 1,
                                      torch.bfloat16)
    small = torch.empty(need1, dtype=torch.uint8, device="cuda:0")
    c = api.search_scale(Xd, Wd, abar, alphas, want_row_sums=True, ws=small)
    for other in (b, c):
        assert np.array_equal(a["mse"], other["mse"])
        assert torch.equal(a["row_sums"], other["row_sums"])
        assert a["index"] == other["index"]


def test_layer512_f32_full(api):
    cfg = synth.CONFIGS["layer512_f32"]
    X, W = synth.make_layer(cfg)
    res, ref, Xd, Wd = check_scale_search(api, X, W, "f32", synth.alpha_grid(cfg.n_alpha), 4, True)
    # fp32 path: E and products stay in float32, so the curve is much tighter
    assert np.max(np.abs(res["mse"] - ref["mse"]) / ref["mse"]) < 1e-5
    check_clip(api, Xd, Wd, X, W, "f32", ref["s_best"], synth.ratio_grid(20), 4, True)


# ---------------------------------------------------------------------------
# step 7: clip search
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits,zp", [(4, True), (3, True), (4, False)])
def test_search_clip_small_ragged(api, bits, zp):
    X, W = synth.make_custom(700, 300, 384, "bf16", seed=31)
    Xd, Wd = to_dev(X, "bf16"), to_dev(W, "bf16")
    ab = O.act_stats(X, "bf16")
    s = O.scale_for_alpha(ab, 0.4)
    check_clip(api, Xd, Wd, X, W, "bf16", s, synth.ratio_grid(6), bits, zp)


# ---------------------------------------------------------------------------
# step 8: pack
# ---------------------------------------------------------------------------

def unpack_codes(words, cols, bits):
    """[R, cols·bits/32] words -> [R, cols] codes; code c at bits bits·c.. of
    the row's little-endian word stream."""
    u = np.ascontiguousarray(words).view(np.uint32).astype(np.uint64)
    out = np.zeros((u.shape[0], cols), dtype=np.int64)
    mask = np.uint64((1 << bits) - 1)
    for c in range(cols):
        w, b = divmod(bits * c, 32)
        v = u[:, w] >> np.uint64(b)
        if b + bits > 32:
            v |= u[:, w + 1] << np.uint64(32 - b)
        out[:, c] = (v & mask).astype(np.int64)
    return out


def assert_pack_parity(qw, qz, sc, W, dtype, s, ratio, zp, bits=4, group=128):
    """GPU packed output against the oracle's; returns the number of near-tie codes."""
    rqw, rqz, rsc, ovf = O.quantize_pack(W, dtype, s, ratio, bits, group, zp)
    assert not ovf
    qw, qz, sc = qw.cpu().numpy(), qz.cpu().numpy(), sc.cpu().numpy().view(np.uint16)
    assert np.array_equal(qz, rqz), "qzeros differ"
    assert np.array_equal(sc, rsc), "scales differ"
    if np.array_equal(qw, rqw):
        return 0
    N = W.shape[0]
    gq, rq = unpack_codes(qw, N, bits), unpack_codes(rqw, N, bits)      # [K, N]
    kk, nn = np.nonzero(gq != rq)
    w32 = O.decode(W, dtype)
    r = np.ones(N, np.float32) if ratio is None else np.asarray(ratio, np.float32)
    _, step, _ = O.quantize(w32[np.unique(nn)], s, r[np.unique(nn)], bits, group, zp)
    row_of = {n: i for i, n in enumerate(np.unique(nn))}
    for k, n in zip(kk, nn):
        wp = np.float32(w32[n, k] * np.float32(s[k]))
        v = float(np.float32(wp / step[row_of[n], k // group]))
        assert abs(v - np.floor(v) - 0.5) < 1e-6, f"code ({k},{n}) differs away from a tie"
        assert abs(int(gq[k, n]) - int(rq[k, n])) == 1
    print(f"pack: {len(kk)} near-tie codes differ")
    return len(kk)


def _pack_case(api, N, K, dtype, zp, with_ratio, seed, bits=4, group=128):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if dtype == "bf16":
        W = synth.f32_to_bf16_bits(w)
    elif dtype == "f16":
        W = w.astype(np.float16).view(np.uint16)
    else:
        W = w
    s = np.exp(rng.uniform(-1.5, 1.5, size=K)).astype(np.float32)
    ratio = rng.choice(synth.ratio_grid(), size=N).astype(np.float32) if with_ratio else None
    qw, qz, sc = api.quantize_pack(to_dev(W, dtype), torch.from_numpy(s).to("cuda:0"),
                                   None if ratio is None else torch.from_numpy(ratio).to("cuda:0"),
                                   bits=bits, group=group, zero_point=zp)
    assert qw.shape == (K, N * bits // 32) and qz.shape == (K // group, N * bits // 32)
    assert sc.shape == (K // group, N)
    assert_pack_parity(qw, qz, sc, W, dtype, s, ratio, zp, bits, group)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("with_ratio", [True, False])
def test_pack_bitwise(api, dtype, zp, with_ratio):
    _pack_case(api, 264, 384, dtype, zp, with_ratio, seed=41)


@pytest.mark.parametrize("N,K", [(8, 128), (256, 128), (520, 256)])
def test_pack_bitwise_shapes(api, N, K):
    _pack_case(api, N, K, "bf16", True, True, seed=N + K)


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("zp", [True, False])
def test_pack_bitwise_bits_groups(api, bits, group, zp):
    # 288 rows: one full 256-row tile and a ragged one (9 x 32 rows for 3 bits)
    _pack_case(api, 288, 384, "bf16", zp, True, seed=bits * 100 + group, bits=bits, group=group)


@pytest.mark.parametrize("N,K", [(32, 128), (544, 256)])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_pack_int3_shapes(api, N, K, dtype):
    _pack_case(api, N, K, dtype, True, False, seed=N * 3 + K, bits=3, group=64)


@pytest.mark.parametrize("bits,group,zp", [(4, 32, True), (4, 64, False), (3, 32, True),
                                           (3, 64, True)])
def test_search_scale_group_sizes(api, bits, group, zp):
    X, W = synth.make_custom(700, 300, 384, "bf16", seed=26 + group)
    check_scale_search(api, X, W, "bf16", synth.alpha_grid(7), bits, zp, group=group)


@pytest.mark.parametrize("bits,group", [(4, 32), (3, 64)])
def test_search_clip_group_sizes(api, bits, group):
    X, W = synth.make_custom(520, 264, 256, "bf16", seed=27 + group)
    ab = O.act_stats(X, "bf16")
    s = O.scale_for_alpha(ab, 0.5)
    check_clip(api, to_dev(X, "bf16"), to_dev(W, "bf16"), X, W, "bf16", s,
               synth.ratio_grid(6), bits, True, group=group)


def test_pack_overflow_reports_range(api):
    from post_weight_quantization_26_amd import _lib
    W = np.where(np.arange(128) % 2 == 0, 1.0, -1.0).astype(np.float32)[None].repeat(8, 0)
    with pytest.raises(_lib.AwqError) as ei:
        api.quantize_pack(to_dev(W, "f32"), torch.full((128,), 1e6, device="cuda:0"))
    assert ei.value.status == _lib.AWQ_E_RANGE
