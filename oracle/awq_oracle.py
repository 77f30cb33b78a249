"""Plain CPU oracle for AWQ's per-layer activation-aware scale search.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
this module: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
cpu_baseline leg use it. It is deliberately slow and literal: each function is
one step of the method as the AWQ pages state it, written with numpy and
float64 accumulation, so a reader can check it against the pages by eye.

Sources (titles of the pages; section names as they appear there):
  [concept]  "AWQ and Activation-Aware Scaling" (concept note).
  [roadmap]  "05 — AWQ: Activation-Aware Weight Scaling" (study roadmap).
  [record]   anthology-of-the-SOTA record SOTA-356, "What to do".

Routes to the output error. ``output_sq_error`` forms X·Eᵀ token block by
token block (the plain definition). ``gram_matrix`` + ``output_sq_error_gram``
form G = XᵀX once and then e·G·eᵀ per row: the same sums in another order,
about T/K times less work for one candidate row, which is what lets the
oracle produce whole error curves of Llama-class layers. Both are pinned
(pure-Python sums; each other to 1e-10).

Precision. Activation statistics, the scale table, the dequantised/folded
weights and every output error are computed in float64. The quantiser itself
(the arithmetic that decides an integer code) runs in IEEE float32 with
round-to-nearest-even, one rounding per operation and no fused multiply-add:
the pages do not fix its precision, and the codes must be decided in the same
precision on both sides of a parity check.

Readings of points the pages leave open (each is listed with its reason in the
project's design notes):
  * ā is the mean of |x| over calibration tokens; ā is floored at 1e-8
    before the power so a dead channel cannot give s = 0.
  * s_j(α) = ā_j^α / sqrt(max_k ā_k^α · min_k ā_k^α), one constant per α.
  * Quantisation groups run along the input dimension, 128 channels each.
  * Min-max range widened to contain 0; asymmetric step (mx-mn)/(2^b-1),
    integer zero point rint(-mn/step) clamped to [0, 2^b-1]; step floored at
    1e-5. Symmetric: step max(|mn|,|mx|)/(2^(b-1)-1), zero point 2^(b-1).
  * code = clamp(rint(w'/step) + zero, 0, 2^b-1); rounding is RNE.
  * A clip ratio r scales the (0-widened) group range to [r·mn, r·mx].
  * The error measure is the mean over tokens and output channels of the
    squared difference of the quantised-and-folded layer's output from the
    exact output of the given inputs.
  * Ties in every argmin go to the lowest grid index.
  * Packing: codes packed densely along the output dimension from the lowest
    bit up (4 bits: 8 per 32-bit word, element 8j+i in bits 4i..4i+3; 3 bits:
    32 per 3 words); zeros packed the same way; scales fp16.
  * Linears that read the same input share one preceding operation, so they
    get one s: their weights are searched as one layer with the outputs
    concatenated, and the error is the mean over all of those outputs.
  * The fold divides the preceding normalisation's per-channel weight (and
    bias, if any), or the preceding linear's output rows and bias, by s:
    one IEEE float32 division per element, rounded once to the storage type.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64


# ----------------------------------------------------------------------------
# Inputs
# ----------------------------------------------------------------------------

def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 values of an input tensor given as bf16 or fp16 bit
    patterns (``uint16``) or as float32."""
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(F32)
    if dtype == "f16":
        return np.asarray(a, dtype=np.uint16).view(np.float16).astype(F32)
    if dtype == "f32":
        return np.asarray(a, dtype=F32)
    raise ValueError(f"unsupported dtype {dtype!r}")


# ----------------------------------------------------------------------------
# Step 1 — activation statistics
# ----------------------------------------------------------------------------

def act_stats(X: np.ndarray, dtype: str, chunk: int = 4096) -> np.ndarray:
    """Per-input-channel mean activation magnitude ā_j = (1/T)·Σ_t |x_tj|.

    [concept] "Scaling instead of protecting": ā is the per-channel mean
    activation magnitude; [roadmap] §4, first step: per-channel activation
    magnitude from the calibration set; [record] "What to do", first item.
    The sum is taken in float64 (token blocks only bound memory) and rounded
    once to float32 after the division by T.
    """
    T, K = X.shape
    S = np.zeros(K, dtype=F64)
    for t0 in range(0, T, chunk):
        x = decode(X[t0:t0 + chunk], dtype).astype(F64)
        S += np.abs(x).sum(axis=0)
    return (S / F64(T)).astype(F32)


# ----------------------------------------------------------------------------
# Step 2 — the scale for each grid exponent
# ----------------------------------------------------------------------------

ABAR_FLOOR = 1e-8


def scale_for_alpha(abar: np.ndarray, alpha: float) -> np.ndarray:
    """s_j = ā_j^α / sqrt(max_k ā_k^α · min_k ā_k^α), float64, rounded once to float32.

    [concept] "Scaling instead of protecting": s = ā^α with α in [0, 1];
    [roadmap] §4: s_j is |X_j|^α times a constant. The constant is taken as
    the reciprocal geometric mean of the largest and smallest scale, so the
    scales straddle 1. α arrives as a float32 grid value.
    """
    a = np.maximum(np.asarray(abar, dtype=F64), F64(ABAR_FLOOR))
    p = a ** F64(F32(alpha))
    s = p / np.sqrt(p.max() * p.min())
    return s.astype(F32)


def scale_table(abar: np.ndarray, alphas) -> np.ndarray:
    """[n_alpha, K] float32 table of ``scale_for_alpha`` over the grid."""
    return np.stack([scale_for_alpha(abar, a) for a in np.asarray(alphas, dtype=F32)])


# ----------------------------------------------------------------------------
# Step 3 — group-wise uniform quantisation of W·diag(s)
# ----------------------------------------------------------------------------

def quant_params(wp_groups: np.ndarray, ratio: np.ndarray, bits: int, zero_point: bool):
    """Step and zero point of each group of scaled weights (float32 arithmetic).

    ``wp_groups`` is [N, G, g] float32 of w' = fl32(w·s). ``ratio`` is [N]
    float32 (1 for no clipping). Returns (step [N, G] float32, zero [N, G]
    float32 holding integers).

    [roadmap] §5: per-group fp16 scales and packed 4-bit zeros along the input
    dimension; §9 option A: zero point on, group 128, 4-bit. The range is the
    group's min and max, widened to contain 0, then scaled by the clip ratio
    ([roadmap] §4 "Optional: per-channel clipping", a fraction 0.5-1.0 of the
    maximum). Symmetric variant: [roadmap] §3 "Why does scaling reduce quant
    error?", a symmetric scheme whose error is at most half a step.
    """
    qmax = F32(2 ** bits - 1)
    mx = np.maximum(wp_groups.max(axis=2), F32(0))
    mn = np.minimum(wp_groups.min(axis=2), F32(0))
    r = np.asarray(ratio, dtype=F32).reshape(-1, 1)
    mx = (r * mx).astype(F32)
    mn = (r * mn).astype(F32)
    if zero_point:
        step = np.maximum((mx - mn) / qmax, F32(1e-5)).astype(F32)
        zero = np.clip(np.rint((-mn) / step), F32(0), qmax).astype(F32)
    else:
        amax = np.maximum(mx, -mn)
        step = np.maximum(amax / F32(2 ** (bits - 1) - 1), F32(1e-5)).astype(F32)
        zero = np.full(step.shape, F32(2 ** (bits - 1)), dtype=F32)
    return step, zero


def quantize(w32: np.ndarray, s32: np.ndarray, ratio, bits: int, group: int,
             zero_point: bool):
    """Codes, steps and zeros of W·diag(s) with groups of ``group`` along the input dim.

    ``w32`` [N, K] float32, ``s32`` [K] float32, ``ratio`` [N] or scalar.
    Returns (q uint8 [N, K], step float32 [N, K/group], zero float32 [N, K/group]).
    Codes: clamp(rint(fl32(w'/step)) + zero, 0, 2^b - 1) ([concept] "Scaling
    instead of protecting": the scaled weight is what is rounded; [record]
    "What to do": round everything uniformly to the target width).
    """
    N, K = w32.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    ratio = np.broadcast_to(np.asarray(ratio, dtype=F32), (N,))
    wp = (w32 * np.asarray(s32, dtype=F32)[None, :]).astype(F32)
    wg = wp.reshape(N, G, group)
    step, zero = quant_params(wg, ratio, bits, zero_point)
    qmax = F32(2 ** bits - 1)
    q = np.clip(np.rint(wg / step[:, :, None]) + zero[:, :, None], F32(0), qmax)
    return q.reshape(N, K).astype(np.uint8), step, zero


# ----------------------------------------------------------------------------
# Step 4 — dequantise and fold diag(s)^-1 back in
# ----------------------------------------------------------------------------

def dequantize(q: np.ndarray, step: np.ndarray, zero: np.ndarray, group: int) -> np.ndarray:
    """Scaled-domain reconstruction (q - zero)·step, float64 [N, K]."""
    N, K = q.shape
    qg = q.reshape(N, K // group, group).astype(F64)
    return ((qg - zero.astype(F64)[:, :, None]) * step.astype(F64)[:, :, None]).reshape(N, K)


def fold(wp_hat: np.ndarray, s32: np.ndarray) -> np.ndarray:
    """Undo the per-input-channel scale: ŵ_nj = ŵ'_nj / s_j (float64).

    [roadmap] §3 "The scaling trick": X·W equals (X·diag(s)^-1)·(diag(s)·W)
    for positive s, so the quantised diag(s)·W acts on X through diag(s)^-1.
    """
    return wp_hat / np.asarray(s32, dtype=F64)[None, :]


# ----------------------------------------------------------------------------
# Step 5 — output error against the unquantised layer
# ----------------------------------------------------------------------------

def output_sq_error(X: np.ndarray, dtype: str, w32: np.ndarray, w_hat: np.ndarray,
                    chunk: int = 8192) -> np.ndarray:
    """M_n = Σ_t (Σ_j x_tj·(ŵ_nj − w_nj))² for each row n of ``w_hat`` (float64).

    This is the squared output difference of the quantised layer from the
    exact product of the given inputs, per output channel, summed over
    tokens ([roadmap] §4: quantise, then measure the output MSE; [concept]
    "Scaling instead of protecting": α minimises reconstruction error).
    ``w_hat`` may hold several candidates stacked along its rows; token
    blocks only bound memory.
    """
    E = np.asarray(w_hat, dtype=F64) - np.asarray(w32, dtype=F64)
    M = np.zeros(E.shape[0], dtype=F64)
    for t0 in range(0, X.shape[0], chunk):
        x = decode(X[t0:t0 + chunk], dtype).astype(F64)
        Y = x @ E.T
        M += (Y * Y).sum(axis=0)
    return M


def gram_matrix(X: np.ndarray, dtype: str, chunk: int = 4096) -> np.ndarray:
    """G = XᵀX over all calibration tokens, float64 [K, K].

    The output error of step 5 is a quadratic form in the error weights:
    Σ_t (Σ_j x_tj·e_j)² = Σ_j Σ_k e_j·(Σ_t x_tj·x_tk)·e_k = e·G·eᵀ. G does
    not depend on the candidate, so it is formed once; token blocks only
    bound memory. (The identity is exact algebra, not a statement of the
    pages; it only reorders the sums of [roadmap] §4's output error.)
    """
    K = X.shape[1]
    G = np.zeros((K, K), dtype=F64)
    for t0 in range(0, X.shape[0], chunk):
        x = decode(X[t0:t0 + chunk], dtype).astype(F64)
        G += x.T @ x
    return G


def output_sq_error_gram(G: np.ndarray, w32: np.ndarray, w_hat: np.ndarray,
                         rows: int = 2048) -> np.ndarray:
    """M_n = e_n·G·e_nᵀ with e_n = ŵ_n − w_n, for each row n of ``w_hat``
    (float64): the same per-row output error as ``output_sq_error``, through
    the Gram matrix of the activations. Row blocks only bound memory."""
    w_hat = np.asarray(w_hat, dtype=F64)
    w = np.asarray(w32, dtype=F64)
    M = np.zeros(w_hat.shape[0], dtype=F64)
    for r0 in range(0, w_hat.shape[0], rows):
        E = w_hat[r0:r0 + rows] - w[r0:r0 + rows]
        M[r0:r0 + rows] = ((E @ G) * E).sum(axis=1)
    return M


def _errors(X, dtype, w, make_candidate, n_cand, G):
    """[n_cand, R] output errors of the candidates ``make_candidate(i)``
    (float64 ŵ, [R, K]) on the rows ``w``: the direct route shares one pass
    over X between all candidates; with G the Gram route takes them one by
    one."""
    if G is None:
        cands = [make_candidate(i) for i in range(n_cand)]
        M = output_sq_error(X, dtype, np.tile(w, (n_cand, 1)), np.concatenate(cands))
        return M.reshape(n_cand, w.shape[0])
    return np.stack([output_sq_error_gram(G, w, make_candidate(i)) for i in range(n_cand)])


# ----------------------------------------------------------------------------
# Steps 2-6 — the α grid search
# ----------------------------------------------------------------------------

def _rows(W, dtype, rows):
    w = decode(W, dtype)
    return w if rows is None else w[np.asarray(rows)]


def candidate_weights(w32, s32, ratio, bits, group, zero_point):
    """Quantised-and-folded weights ŵ for one candidate (float64 [N, K])."""
    q, step, zero = quantize(w32, s32, ratio, bits, group, zero_point)
    return fold(dequantize(q, step, zero, group), s32)


def search_scale(X, W, dtype, abar, alphas, bits=4, group=128, zero_point=True, rows=None,
                 G=None):
    """Grid search over α ([roadmap] §4; [concept] "Scaling instead of protecting").

    For each grid value: scale, quantise, fold back and measure the output
    error. Returns a dict with ``row_sums`` [n_alpha, R] (M_n per candidate for
    the R selected rows, all rows by default), ``mse`` [n_alpha] =
    Σ_n M_n / (T·R), ``index`` (argmin, lowest index on ties), ``alpha_best``,
    ``s_best`` and the whole ``s_table``. With a row subset the curve is that
    subset's; the chosen α is then the subset's too. With ``G`` (the
    ``gram_matrix`` of X) the errors come from the Gram route; X is then
    used only for its token count.
    """
    alphas = np.asarray(alphas, dtype=F32)
    T = X.shape[0]
    w = _rows(W, dtype, rows)
    s_tab = scale_table(abar, alphas)
    R = w.shape[0]
    row_sums = _errors(X, dtype, w,
                       lambda i: candidate_weights(w, s_tab[i], 1.0, bits, group, zero_point),
                       len(alphas), G)
    mse = row_sums.sum(axis=1) / F64(T * R)
    best = int(np.argmin(mse))
    return dict(row_sums=row_sums, mse=mse, index=best, alpha_best=F32(alphas[best]),
                s_best=s_tab[best].copy(), s_table=s_tab)


# ----------------------------------------------------------------------------
# Step 7 — per-output-channel clip-ratio search
# ----------------------------------------------------------------------------

def search_clip(X, W, dtype, s32, ratios, bits=4, group=128, zero_point=True, rows=None,
                G=None):
    """Per-output-channel clip search with s fixed ([roadmap] §4 "Optional:
    per-channel clipping": after α is picked, a clip ratio between 0.5 and
    1.0 of the maximum is searched per channel).

    Every group of row n uses that row's ratio. Row n's output error depends
    only on row n, so the per-row argmin is the joint optimum. Returns
    ``row_sums`` [n_ratio, R], ``index`` [R], ``ratio_best`` [R] and
    ``mse_clip`` = Σ_n M_n(r*_n) / (T·R). ``G`` selects the Gram route, as
    in ``search_scale``.
    """
    ratios = np.asarray(ratios, dtype=F32)
    T = X.shape[0]
    w = _rows(W, dtype, rows)
    R = w.shape[0]
    row_sums = _errors(X, dtype, w,
                       lambda i: candidate_weights(w, s32, np.full(R, ratios[i], dtype=F32),
                                                   bits, group, zero_point),
                       len(ratios), G)
    idx = np.argmin(row_sums, axis=0)
    mse_clip = row_sums[idx, np.arange(R)].sum() / F64(T * R)
    return dict(row_sums=row_sums, index=idx, ratio_best=ratios[idx], mse_clip=F64(mse_clip))


# ----------------------------------------------------------------------------
# Step 8 — quantise and pack
# ----------------------------------------------------------------------------

def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """[R, C] codes of ``bits`` bits -> [R, C·bits/32] int32, packed densely
    along each row from the lowest bit up: element c occupies bits
    bits·c .. bits·c + bits - 1 of the row's little-endian bit stream, so a
    code may straddle two words. For 4 bits this is 8 codes per word, element
    8j+i in bits 4i..4i+3 of word j, as [roadmap] §5 prints; 3 bits fill
    3 words with 32 codes."""
    R, C = codes.shape
    if (C * bits) % 32:
        raise ValueError("a row must fill whole 32-bit words")
    v = codes.astype(np.uint64)
    out = np.zeros((R, C * bits // 32), dtype=np.uint64)
    for c in range(C):
        w, b = divmod(bits * c, 32)
        out[:, w] |= (v[:, c] << np.uint64(b)) & np.uint64(0xFFFFFFFF)
        if b + bits > 32:
            out[:, w + 1] |= v[:, c] >> np.uint64(32 - b)
    return out.astype(np.uint32).view(np.int32)


def quantize_pack(W, dtype, s32, ratio=None, bits=4, group=128, zero_point=True):
    """Packed layer in the AWQ storage layout ([roadmap] §5), 4 or 3 bits.

    qweight [K, N·b/32] int32 (input-major, codes packed along the output
    dim), qzeros [K/g, N·b/32] int32 packed the same way, scales [K/g, N] fp16
    bits (RNE of the float32 step). The codes represent W·diag(s), clipped by
    ``ratio`` per row; the caller folds diag(s)^-1 into the preceding
    operation. Returns (qweight, qzeros, scales_u16, overflow_flag).
    """
    if bits not in (3, 4):
        raise ValueError("packing is defined for 3- and 4-bit codes")
    w = decode(W, dtype)
    N, K = w.shape
    if (N * bits) % 32:
        raise ValueError("N·bits must be a multiple of 32")
    r = np.ones(N, dtype=F32) if ratio is None else np.asarray(ratio, dtype=F32)
    q, step, zero = quantize(w, s32, r, bits, group, zero_point)
    qweight = pack_codes(np.ascontiguousarray(q.T), bits)
    qzeros = pack_codes(np.ascontiguousarray(zero.astype(np.uint8).T), bits)
    with np.errstate(over="ignore"):
        sc = step.T.astype(np.float16)
    overflow = bool(~np.isfinite(sc).all())
    return qweight, qzeros, np.ascontiguousarray(sc).view(np.uint16), overflow


def unpack_codes(words: np.ndarray, count: int, bits: int) -> np.ndarray:
    """Inverse of ``pack_codes``: [R, W] int32 words -> [R, count] codes, code c
    read from bits bits·c .. bits·c + bits - 1 of the row's little-endian
    stream of words."""
    u = np.ascontiguousarray(words).view(np.uint32).astype(np.uint64)
    out = np.zeros((u.shape[0], count), dtype=np.int64)
    mask = np.uint64((1 << bits) - 1)
    for c in range(count):
        w, b = divmod(bits * c, 32)
        v = u[:, w] >> np.uint64(b)
        if b + bits > 32:
            v = v | (u[:, w + 1] << np.uint64(32 - b))
        out[:, c] = (v & mask).astype(np.int64)
    return out


def dequantize_packed(qweight, qzeros, scales_u16, N: int, bits: int = 4, group: int = 128):
    """Weights a consumer of the packed layout sees, float64 [N, K]:
    ŵ[n][k] = (q[k][n] - z[k/g][n]) · scale[k/g][n], with the stored fp16
    scale ([roadmap] §5: qweight, qzeros and fp16 scales; §3: these are the
    weights of W·diag(s), to be applied to X·diag(s)^-1)."""
    q = unpack_codes(qweight, N, bits)                        # [K, N]
    z = unpack_codes(qzeros, N, bits)                         # [K/g, N]
    sc = np.asarray(scales_u16, dtype=np.uint16).view(np.float16).astype(F64)   # [K/g, N]
    K = q.shape[0]
    gidx = np.arange(K) // group
    return ((q - z[gidx]).astype(F64) * sc[gidx]).T           # [N, K]


def w4a16_matmul(Xp, dtype, qweight, qzeros, scales_u16, N: int, bits: int = 4,
                 group: int = 128) -> np.ndarray:
    """Y = X'·Ŵᵀ in float64 for activations X' [T, K] (already divided by s,
    the fold) and a packed layer: what a weight-only-quantised (W4A16) layer
    computes ([reading] "Key takeaways": weight-only INT4 with 16-bit
    activations; [roadmap] §5 for the format)."""
    x = decode(Xp, dtype).astype(F64)
    return x @ dequantize_packed(qweight, qzeros, scales_u16, N, bits, group).T


def storage_bits_per_weight(N: int, K: int, bits: int = 4, group: int = 128) -> float:
    """Bits per weight of the packed layout: codes + fp16 scales + packed zeros."""
    total = N * K * bits + (N * K // group) * (16 + bits)
    return total / (N * K)


# ----------------------------------------------------------------------------
# Linears sharing one input, and the fold of diag(s)^-1 into the op before
# ([concept] "Scaling instead of protecting": the division of the activation
# channel goes into the preceding layer, usually the normalisation's scale;
# "When it breaks": that op must be a norm or a linear with per-channel
# weights)
# ----------------------------------------------------------------------------

def search_scale_group(X, Ws, dtype, abar, alphas, bits=4, group=128, zero_point=True, rows=None,
                       G=None):
    """α search for several linears that read the same X (for example the
    query, key and value projections after one normalisation).

    Only one op precedes them, so one s must serve them all. Their outputs,
    side by side, are the group's output; its error is measured over all of
    them, which is the single-layer search of the weights stacked along the
    output dimension. ``rows`` index the stacked rows. Same result dict as
    ``search_scale``.
    """
    W = np.concatenate([np.asarray(w) for w in Ws], axis=0)
    return search_scale(X, W, dtype, abar, alphas, bits, group, zero_point, rows=rows, G=G)


def encode(v32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> storage of ``dtype`` (bf16/f16 as uint16 bit
    patterns), rounded to the nearest representable value, ties to the even
    significand; values past the largest finite one round to infinity as
    IEEE rounding prescribes."""
    v = np.ascontiguousarray(v32, dtype=F32)
    if dtype == "f32":
        return v.copy()
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return v.astype(np.float16).view(np.uint16)      # IEEE conversion, ties to even
    if dtype != "bf16":
        raise ValueError(f"unsupported dtype {dtype!r}")
    u = v.view(np.uint32)
    lo = (u >> np.uint32(16)).astype(np.uint32)              # same sign, magnitude truncated
    exp = (lo >> np.uint32(7)) & np.uint32(0xFF)
    # one unit in the last place of a bf16 with this exponent field (8 significand bits)
    ulp = np.ldexp(1.0, np.maximum(exp.astype(np.int64), 1) - 127 - 7)
    x = np.abs(v.astype(F64))
    x_lo = np.abs((lo << np.uint32(16)).view(F32).astype(F64))
    finite = np.isfinite(v)
    with np.errstate(invalid="ignore"):
        d_lo = x - x_lo
        d_hi = (x_lo + ulp) - x
    up = finite & ((d_hi < d_lo) | ((d_hi == d_lo) & ((lo & np.uint32(1)) == 1)))
    out = np.where(up, lo + np.uint32(1), lo)
    nan = np.isnan(v)
    out = np.where(nan, out | np.uint32(0x0040), out)         # keep NaN a (quiet) NaN
    return out.astype(np.uint16)


def _divide_stored(a, dtype, d32):
    """fl32(a / d) elementwise (numpy's float32 division is IEEE's correctly
    rounded quotient), stored back as ``dtype``."""
    with np.errstate(over="ignore", under="ignore"):
        q = decode(a, dtype) / np.asarray(d32, dtype=F32)
    return encode(q.astype(F32), dtype)


def fold_norm(gamma, beta, dtype, s32):
    """Normalisation before the layer: y_j = γ_j·x̂_j (+ β_j). Dividing
    activation channel j by s_j is γ_j / s_j (and β_j / s_j). Returns
    (γ', β' or None) in the storage ``dtype``."""
    s = np.asarray(s32, dtype=F32)
    g = _divide_stored(gamma, dtype, s)
    b = None if beta is None else _divide_stored(beta, dtype, s)
    return g, b


def fold_linear(W_prev, b_prev, dtype, s32):
    """Linear before the layer: h = x·W_prevᵀ + b_prev with W_prev [K, K_prev];
    output channel j of h is input channel j of the layer, so row j of W_prev
    and b_prev[j] are divided by s_j. Returns (W_prev', b_prev' or None)."""
    s = np.asarray(s32, dtype=F32)
    W = _divide_stored(W_prev, dtype, s[:, None])
    b = None if b_prev is None else _divide_stored(b_prev, dtype, s)
    return W, b
