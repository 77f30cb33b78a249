/*
 * awq.h — C ABI of the AWQ per-layer activation-aware scale search on MI355X.
 *
 * For one linear layer Y = X·Wᵀ (X [T, K] calibration activations, W [N, K]
 * weights, K input channels, N output channels) the library computes:
 *
 *   awq_act_stats      ā_j = mean_t |x_tj|                       (step 1)
 *   awq_act_stats_accumulate / _finalize   the same over calibration batches
 *   awq_scale_table    s_j(α) = ā_j^α / sqrt(max ā^α · min ā^α)  (step 2)
 *   awq_search_scale   for each α of a grid: quantise W·diag(s) group-wise,
 *                      fold diag(s)^-1 back, measure the output MSE against
 *                      the unquantised product; return the curve and argmin
 *   awq_search_clip    per-output-channel clip ratio search with s fixed
 *   awq_quantize_pack  INT4 or INT3 codes, packed zeros and fp16 scales
 *   awq_search_scale_group  the α search for several linears that read the
 *                      same X and so share one s
 *   awq_fold_norm, awq_fold_linear  divide the operation that produces X by
 *                      s, so the scaled weights need no run-time division
 *   awq_w4a16_matmul   a consumer of the packed layout: Y = X·Ŵᵀ
 *
 * Sources (page titles and sections):
 *   "AWQ and Activation-Aware Scaling", section "Scaling instead of
 *   protecting" — s = ā^α with α in [0, 1] found by a per-layer grid search
 *   minimising reconstruction error; α = 0 is plain quantisation.
 *   "05 — AWQ: Activation-Aware Weight Scaling": section 3 "The scaling
 *   trick" (the invariance X·W = (X·diag(s)^-1)(diag(s)·W)); section 4 "How
 *   to find s — the grid search" (~20 α values in [0, 1], output MSE, pick
 *   the best) and "Optional: per-channel clipping" (ratios 0.5–1.0 of the
 *   max after α is chosen); section 5 "Bit-level output format" (qweight,
 *   qzeros, scales layout); section 9 option A (zero point, group 128, 4 bit).
 *   Anthology record SOTA-356, "What to do" (collect per-input-channel
 *   activation statistics, scale, round uniformly).
 *
 * Conventions for every entry point:
 *   - Arrays are DEVICE pointers unless marked [host]. Matrices are dense and
 *     row-major. The caller owns and allocates every buffer; the library
 *     keeps no device memory between calls (workspaces are passed in).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All device work is enqueued on it in order. Functions with [host]
 *     outputs synchronise `stream` before returning; the others do not.
 *   - Arguments are validated on the host before anything is enqueued. A
 *     failed check returns a negative status and launches nothing.
 *     X and W must be 16-byte aligned; K must be a multiple of 128 (for
 *     every group size); grids hold 1..64 values. Sizes past the kernels'
 *     32-bit offsets and grids return AWQ_E_UNSUPPORTED: 16-bit searches and
 *     the consumer need 512·K < 2^31 (split candidates: 512·2K < 2^31),
 *     weight matrices at most 2^34 elements, and one batch of the candidate
 *     GEMM fewer than 2^32 work-items (a search takes smaller batches
 *     where that is what keeps it within the grid).
 *   - Quantiser arithmetic is IEEE float32 with round-to-nearest-even, one
 *     rounding per operation (no contraction, no flush of denormals):
 *       w' = w·s_j; mx = r·max(0, max_G w'); mn = r·min(0, min_G w')
 *       asymmetric: step = max((mx-mn)/(2^b-1), 1e-5);
 *                   zero = clamp(rint(-mn/step), 0, 2^b-1)
 *       symmetric:  step = max(max(mx,-mn)/(2^(b-1)-1), 1e-5); zero = 2^(b-1)
 *       code = clamp(rint(w'/step) + zero, 0, 2^b-1)
 *     Groups are g consecutive input channels of one output row, g = 32, 64
 *     or 128 (AutoAWQ's q_group_size; 128 in the pages' configuration).
 *   - Errors never abort: a non-zero status is returned and
 *     awq_last_error() describes it (per calling thread).
 *   - Calls are thread-compatible: concurrent calls must use distinct
 *     workspaces.
 */
#ifndef AWQ_MI355X_AWQ_H
#define AWQ_MI355X_AWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AWQ_OK = 0,
  AWQ_E_INVALID = -1,     /* bad argument: shape, NULL, alignment, grid value */
  AWQ_E_UNSUPPORTED = -2, /* valid but not implemented (dtype, bits, group) */
  AWQ_E_WORKSPACE = -3,   /* workspace smaller than the minimum */
  AWQ_E_RANGE = -4,       /* a result is out of range: an fp16 scale overflowed in
                             awq_quantize_pack, or a search's output error is not
                             finite (NaN or Inf in its inputs) */
  AWQ_E_HIP = -5          /* a HIP runtime call failed (message in awq_last_error) */
} awq_status;

typedef enum { AWQ_F32 = 0, AWQ_BF16 = 1, AWQ_F16 = 2 } awq_dtype;

/* Quantiser parameters. w_bit: 4 or 3. group_size: 32, 64 or 128.
 * zero_point: 1 = asymmetric min-max with an integer zero point,
 * 0 = symmetric (zero point fixed at 2^(w_bit-1)).
 * flags: 0, or AWQ_SEARCH_SPLIT_E for the direct searches (awq_search_scale,
 * awq_search_clip, awq_search_scale_group) on bf16 or fp16 layers: each
 * candidate's error weight e = ŵ - w goes to the matrix cores as two 16-bit
 * halves, hi = rnd(e) and lo = rnd(e - hi), instead of one rounding. The
 * per-row output errors then carry only float32 accumulation error (about
 * 16 significand bits in the operand instead of 8 for bf16 or 11 for fp16),
 * for twice the search GEMM's work and twice its candidate buffer (size the
 * workspace with AWQ_OP_SEARCH_SCALE_SPLIT_E / AWQ_OP_SEARCH_CLIP_SPLIT_E).
 * Float32 layers already use float32 operands and ignore the flag; the Gram
 * searches reject it (AWQ_E_UNSUPPORTED); awq_quantize_pack ignores it.
 * Or AWQ_SEARCH_FUSED for awq_search_scale and awq_search_clip on bf16 or
 * fp16 layers with N a multiple of 256 ("05 — AWQ" section 4, the scale /
 * quantise / measure steps in one pass): no candidate buffer is written;
 * a parameter pass stores each (candidate, row, group)'s step, zero point
 * and reciprocal, and the search GEMM forms the candidates' error weights
 * while it stages its operand. The results equal those of flags = 0 bit for
 * bit. The candidate buffer shrinks from 2K to K/2 bytes per candidate row
 * (size the workspace with AWQ_OP_SEARCH_SCALE_FUSED /
 * AWQ_OP_SEARCH_CLIP_FUSED; the plain ops' larger sizes work too); the
 * search GEMM runs about 1.9 times as long. Every other search, float32
 * layers, other N and the combination with AWQ_SEARCH_SPLIT_E are rejected
 * (AWQ_E_UNSUPPORTED). */
typedef struct {
  int32_t w_bit;
  int32_t group_size;
  int32_t zero_point;
  int32_t flags;
} awq_qconfig;

enum { AWQ_SEARCH_SPLIT_E = 1, AWQ_SEARCH_FUSED = 2 };

enum { AWQ_OP_STATS = 0, AWQ_OP_SEARCH_SCALE = 1, AWQ_OP_SEARCH_CLIP = 2, AWQ_OP_PACK = 3,
       AWQ_OP_SEARCH_SCALE_GRAM = 4, AWQ_OP_SEARCH_CLIP_GRAM = 5,
       /* awq_gram_build, and the Gram searches that take a prepared G */
       AWQ_OP_GRAM_BUILD = 6, AWQ_OP_SEARCH_SCALE_GRAM_G = 7, AWQ_OP_SEARCH_CLIP_GRAM_G = 8,
       /* the direct searches with qc.flags = AWQ_SEARCH_SPLIT_E (bf16, fp16) */
       AWQ_OP_SEARCH_SCALE_SPLIT_E = 9, AWQ_OP_SEARCH_CLIP_SPLIT_E = 10,
       /* the direct searches with qc.flags = AWQ_SEARCH_FUSED (bf16, fp16) */
       AWQ_OP_SEARCH_SCALE_FUSED = 11, AWQ_OP_SEARCH_CLIP_FUSED = 12 };

/* Workspace bytes that let `op` process all `n_grid` candidates in one
 * batch (the fastest configuration). Returns 0 for invalid sizes. Pure host
 * arithmetic. */
size_t awq_workspace_bytes(int op, int64_t T, int64_t N, int64_t K, int32_t n_grid,
                           awq_dtype dtype);

/* Workspace bytes for a search (AWQ_OP_SEARCH_SCALE / AWQ_OP_SEARCH_CLIP and
 * their _SPLIT_E, _FUSED and Gram forms)
 * that works through its `n_grid` candidates in batches of at most `batch`
 * (1 <= batch <= n_grid; batch 1 is the minimum any search call accepts).
 * A search call picks the largest batch its workspace allows; results do not
 * depend on the batch. Returns 0 for invalid arguments. */
size_t awq_workspace_bytes_batch(int op, int64_t T, int64_t N, int64_t K, int32_t n_grid,
                                 int32_t batch, awq_dtype dtype);

/* Step 1 — per-input-channel mean activation magnitude.
 * X [T, K] (bf16, f16 or f32) -> abar [K] f32 with abar_j = fl32(Σ_t |x_tj| / T),
 * the sum taken in float64. K must be a multiple of 8 (f32: of 4).
 * Does not synchronise. */
awq_status awq_act_stats(const void* X, awq_dtype x_dtype, int64_t T, int64_t K, float* abar,
                         void* ws, size_t ws_bytes, void* stream);

/* awq_act_stats without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). It allocates nothing: the float64 partials go to a
 * static device array of 2^20 doubles (8 MiB) that each GPU the library runs
 * on holds until the process ends, found once per device on its first call
 * there (the current device must be the one `stream` belongs to). Results
 * equal awq_act_stats bit for bit. Every call on a GPU shares that GPU's
 * array, so calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller. Sizes whose partials need more than
 * 2^20 doubles (awq_workspace_bytes(AWQ_OP_STATS, ...) > 8 MiB, i.e. K above
 * 2^20) return AWQ_E_UNSUPPORTED; other argument errors as
 * for awq_act_stats. Does not synchronise. */
awq_status awq_act_stats_noalloc(const void* X, awq_dtype x_dtype, int64_t T, int64_t K,
                                 float* abar, void* stream);

/* Step 1 over a calibration set that comes in batches: ā is the mean over
 * all their tokens (the statistic is a plain mean, so batches add up).
 * awq_act_stats_accumulate adds Σ_t |x_tj| of one batch X [T, K] (bf16, f16
 * or f32; K as for awq_act_stats) to sums[j]: sums [K] float64 on the
 * device, owned by the caller, zeroed by the caller before the first batch.
 * Batches may differ in T; their order fixes the float64 rounding (a single
 * batch gives exactly awq_act_stats's sum). Workspace as for awq_act_stats
 * with this batch's T (awq_workspace_bytes(AWQ_OP_STATS, T, 1, K, 1, dtype)).
 * awq_act_stats_finalize writes abar_j = fl32(sums_j / count), count = the
 * total number of tokens (>= 1). Neither synchronises; calls on one stream
 * run in order. Errors: AWQ_E_INVALID for NULL or misaligned pointers (sums
 * 8-byte, abar 4-byte) or bad sizes, AWQ_E_WORKSPACE as for awq_act_stats. */
awq_status awq_act_stats_accumulate(const void* X, awq_dtype x_dtype, int64_t T, int64_t K,
                                    double* sums, void* ws, size_t ws_bytes, void* stream);
awq_status awq_act_stats_finalize(const double* sums, int64_t count, int64_t K, float* abar,
                                  void* stream);

/* Step 2 — scale table s[a][j] = ā_j^α_a / sqrt(max_k ā_k^α_a · min_k ā_k^α_a),
 * computed in float64 and rounded once to f32; ā is floored at 1e-8.
 * abar [K] f32; alphas [host] n_alpha values in [0, 1]; s_table [n_alpha, K].
 * Does not synchronise. */
awq_status awq_scale_table(const float* abar, int64_t K, const float* alphas, int32_t n_alpha,
                           float* s_table, void* stream);

/* Steps 2-6 — α grid search for one layer.
 * X [T, K], W [N, K] of `dtype` (bf16, fp16 or f32; the candidates' error
 * weights go to the GEMM in the same type); abar [K] from awq_act_stats;
 * alphas [host] n_alpha values in [0, 1].
 * Outputs: s_best [K] f32 = the scale row of the best α;
 *          alpha_best [host] 1 f32; mse [host] n_alpha f64, mse[a] =
 *          Σ_{t,n} (Y_a - Y)_{tn}² / (T·N) where Y_a uses the quantised,
 *          folded weights; row_sums [n_alpha, N] f64 (per output channel
 *          Σ_t, optional: may be NULL). Ties go to the lowest index.
 * Synchronises `stream`. Returns AWQ_E_RANGE if a curve value is not finite
 * (the curve is written; s_best and alpha_best are not). */
awq_status awq_search_scale(const void* X, const void* W, awq_dtype dtype, int64_t T, int64_t N,
                            int64_t K, const float* abar, const float* alphas, int32_t n_alpha,
                            awq_qconfig qc, float* s_best, float* alpha_best, double* mse,
                            double* row_sums, void* ws, size_t ws_bytes, void* stream);

/* Step 7 — per-output-channel clip-ratio search with s fixed.
 * s [K] f32 (normally s_best); ratios [host] n_ratio values in (0, 1].
 * Every group of row n uses ratio r_n. Outputs: ratio_best [N] f32 (argmin
 * per row, lowest index on ties); mse_clip [host] 1 f64 = Σ_n min_r M_n(r) / (T·N);
 * row_sums [n_ratio, N] f64 = M_n(r) (optional: may be NULL).
 * Synchronises `stream`. Returns AWQ_E_RANGE if mse_clip is not finite. */
awq_status awq_search_clip(const void* X, const void* W, awq_dtype dtype, int64_t T, int64_t N,
                           int64_t K, const float* s, const float* ratios, int32_t n_ratio,
                           awq_qconfig qc, float* ratio_best, double* mse_clip, double* row_sums,
                           void* ws, size_t ws_bytes, void* stream);

/* Step 8 — quantise W·diag(s) (rows clipped by `ratio`, NULL = 1) and pack
 * ("05 — AWQ", section 5 "Bit-level output format").
 * W [N, K] (bf16, f16 or f32); b = w_bit (4 or 3); g = group_size.
 * Codes are packed densely along the output dim from the lowest bit up: in
 * row k of qweight [K, N·b/32] int32, the code of output row n occupies bits
 * b·n .. b·n+b-1 of the little-endian stream of the row's words. For b = 4
 * (N a multiple of 8) word (k, j) holds rows 8j..8j+7, row 8j+i in bits
 * 4i..4i+3, the pages' layout; for b = 3 (N a multiple of 32) 32 rows fill
 * 3 words and rows 10 and 21 of each 32 straddle two words.
 * qzeros [K/g, N·b/32] int32 packed the same way. scales [K/g, N] IEEE fp16
 * bits (RNE of the f32 step).
 * The codes represent W·diag(s); the caller folds diag(s)^-1 into the
 * operation that produces X. ws: at least awq_workspace_bytes(AWQ_OP_PACK,...).
 * N must keep 64·N below 2^31 (AWQ_E_UNSUPPORTED otherwise).
 * Synchronises `stream`; returns AWQ_E_RANGE if a scale overflowed fp16. */
awq_status awq_quantize_pack(const void* W, awq_dtype w_dtype, int64_t N, int64_t K,
                             const float* s, const float* ratio, awq_qconfig qc, int32_t* qweight,
                             int32_t* qzeros, uint16_t* scales, void* ws, size_t ws_bytes,
                             void* stream);

/* The same two searches through the Gram matrix G = XᵀX of the activations:
 * M_n = Σ_t (X·E_nᵀ)_t² = E_n·G·E_nᵀ, an exact identity of the error measure
 * ("05 — AWQ", section 4; the identity itself is not on the pages). G is
 * built once per call (its upper 256x256 tiles, T·K·(K + 256) flops, stored
 * as two bf16 halves hi + lo), then each candidate row costs about
 * 2·K·(K + 256) flops (G's diagonal tiles and twice its upper tiles, over hi
 * and lo) instead of 2·T·K: ~15x fewer at 64K tokens and K = 4096. The
 * candidates' error weights are
 * the same bf16 operands as on the direct path; only the float32 rounding
 * order of the sums differs. Arguments, outputs and synchronisation as in
 * awq_search_scale / awq_search_clip; bf16 inputs only; K below about 2^21
 * (512·(2K + 256) < 2^31), else AWQ_E_UNSUPPORTED. The build reads X as it
 * is (no transposed copy). The workspace (awq_workspace_bytes with
 * AWQ_OP_SEARCH_SCALE_GRAM / AWQ_OP_SEARCH_CLIP_GRAM) also holds the
 * build's float32 partial tiles (up to 16 token slices of G's upper 256x256
 * tiles) and G's upper tiles as bf16 hi/lo halves (K x (2K + 256)
 * elements). */
awq_status awq_search_scale_gram(const void* X, const void* W, awq_dtype dtype, int64_t T,
                                 int64_t N, int64_t K, const float* abar, const float* alphas,
                                 int32_t n_alpha, awq_qconfig qc, float* s_best,
                                 float* alpha_best, double* mse, double* row_sums, void* ws,
                                 size_t ws_bytes, void* stream);
awq_status awq_search_clip_gram(const void* X, const void* W, awq_dtype dtype, int64_t T,
                                int64_t N, int64_t K, const float* s, const float* ratios,
                                int32_t n_ratio, awq_qconfig qc, float* ratio_best,
                                double* mse_clip, double* row_sums, void* ws, size_t ws_bytes,
                                void* stream);

/* Steps 2-6 for a group of linears that read the same X (e.g. the query,
 * key and value projections after one normalisation, or the gate and up
 * projections). The division by s can go into only one preceding operation,
 * so the group gets one s ("AWQ and Activation-Aware Scaling", section
 * "Scaling instead of protecting", the fold into the preceding layer). The
 * group's output is its layers' outputs side by side, and the error is
 * averaged over all of them:
 *   mse[a] = Σ_l Σ_{t,n} (Y_l,a - Y_l)_{tn}² / (T·Σ_l N[l]).
 * W [host] n_layers device pointers to [N[l], K] weights (16-byte aligned);
 * N [host] n_layers output-channel counts; 1 <= n_layers <= 16.
 * row_sums (optional) is [n_alpha, Σ_l N[l]] with the layers' rows in order.
 * The workspace is sized as for awq_search_scale with N = Σ_l N[l]. Every
 * other argument and output is as in awq_search_scale, which this equals
 * when n_layers is 1. Synchronises `stream`. */
awq_status awq_search_scale_group(const void* X, const void* const* W, const int64_t* N,
                                  int32_t n_layers, awq_dtype dtype, int64_t T, int64_t K,
                                  const float* abar, const float* alphas, int32_t n_alpha,
                                  awq_qconfig qc, float* s_best, float* alpha_best, double* mse,
                                  double* row_sums, void* ws, size_t ws_bytes, void* stream);

/* The group search through the Gram matrix of the shared X (as
 * awq_search_scale_gram is to awq_search_scale): one G serves every layer of
 * the group. Arguments and outputs as in awq_search_scale_group; bf16 inputs
 * only; workspace sized with AWQ_OP_SEARCH_SCALE_GRAM and N = Σ_l N[l]. */
awq_status awq_search_scale_group_gram(const void* X, const void* const* W, const int64_t* N,
                                       int32_t n_layers, awq_dtype dtype, int64_t T, int64_t K,
                                       const float* abar, const float* alphas, int32_t n_alpha,
                                       awq_qconfig qc, float* s_best, float* alpha_best,
                                       double* mse, double* row_sums, void* ws, size_t ws_bytes,
                                       void* stream);

/* The consumer of the 3-bit layout (awq_quantize_pack with w_bit = 3): as
 * awq_w4a16_matmul, with qweight [K, N·3/32] and qzeros [K/g, N·3/32] packed
 * densely (N a multiple of 32). T <= 16: the matrix-core decode of
 * awq_w4a16_matmul on the exact Ŵ = (q - z)·scale (the workspace holds the
 * float32 partials). T > 16: Ŵ is formed in float32 and rounded once to the
 * activation type into the workspace (N·K 16-bit values), then the MFMA GEMM
 * computes Y. awq_w3a16_workspace_bytes gives the size for each T. Errors and
 * synchronisation as for awq_w4a16_matmul. */
size_t awq_w3a16_workspace_bytes(int64_t T, int64_t N, int64_t K, awq_dtype dtype);
awq_status awq_w3a16_matmul(const void* X, awq_dtype dtype, int64_t T, int64_t N, int64_t K,
                            const int32_t* qweight, const int32_t* qzeros,
                            const uint16_t* scales, int32_t group_size, void* Y, void* ws,
                            size_t ws_bytes, void* stream);

/* One Gram matrix for every search of the layers that read the same X: the
 * scale search, the clip searches that follow it, and group searches.
 * awq_gram_build writes G of X [T, K] (bf16, K a multiple of 128, T and K
 * within the Gram searches' limits)
 * into G, a caller-owned device buffer of at least awq_gram_bytes(K) bytes
 * (16-byte aligned), in the layout the Gram searches read (G's upper tiles as
 * bf16 hi/lo halves; the rest of the buffer is not written). Workspace:
 * awq_workspace_bytes(AWQ_OP_GRAM_BUILD, T, 1, K, 1, AWQ_BF16). Does not
 * synchronise. awq_gram_bytes returns 0 for K not a multiple of 128.
 * The _g searches take G in place of X and otherwise equal awq_search_scale_gram,
 * awq_search_clip_gram and awq_search_scale_group_gram, bit for bit; T is
 * the token count G was built from. Their workspaces
 * (AWQ_OP_SEARCH_SCALE_GRAM_G, AWQ_OP_SEARCH_CLIP_GRAM_G; N = Σ_l N[l] for
 * a group) hold no partial tiles and no G. Errors as for the searches they replace;
 * AWQ_E_WORKSPACE also when G_bytes < awq_gram_bytes(K). */
size_t awq_gram_bytes(int64_t K);
awq_status awq_gram_build(const void* X, awq_dtype dtype, int64_t T, int64_t K, void* G,
                          size_t G_bytes, void* ws, size_t ws_bytes, void* stream);
awq_status awq_search_scale_gram_g(const void* G, const void* W, awq_dtype dtype, int64_t T,
                                   int64_t N, int64_t K, const float* abar, const float* alphas,
                                   int32_t n_alpha, awq_qconfig qc, float* s_best,
                                   float* alpha_best, double* mse, double* row_sums, void* ws,
                                   size_t ws_bytes, void* stream);
awq_status awq_search_clip_gram_g(const void* G, const void* W, awq_dtype dtype, int64_t T,
                                  int64_t N, int64_t K, const float* s, const float* ratios,
                                  int32_t n_ratio, awq_qconfig qc, float* ratio_best,
                                  double* mse_clip, double* row_sums, void* ws, size_t ws_bytes,
                                  void* stream);
awq_status awq_search_scale_group_gram_g(const void* G, const void* const* W, const int64_t* N,
                                         int32_t n_layers, awq_dtype dtype, int64_t T, int64_t K,
                                         const float* abar, const float* alphas, int32_t n_alpha,
                                         awq_qconfig qc, float* s_best, float* alpha_best,
                                         double* mse, double* row_sums, void* ws,
                                         size_t ws_bytes, void* stream);

/* The fold into a preceding normalisation ("AWQ and Activation-Aware
 * Scaling", sections "Scaling instead of protecting" and "When it breaks").
 * In place: gamma[j] <- gamma[j] / s[j] and, when beta is not NULL,
 * beta[j] <- beta[j] / s[j], for j < K. Each value is converted to float32,
 * divided once (IEEE float32) and rounded once, to nearest even, back to
 * `dtype` (bf16, f16 or f32). gamma, beta: [K] device arrays aligned to
 * their element size; s: [K] f32 (normally s_best). Does not synchronise. */
awq_status awq_fold_norm(void* gamma, void* beta, awq_dtype dtype, int64_t K, const float* s,
                         void* stream);

/* The fold into a preceding linear layer h = x·W_prevᵀ + b_prev whose K
 * output channels are this layer's K input channels (same sections as
 * awq_fold_norm). In place: row j of W_prev [K, K_prev] and bias_prev[j]
 * (when not NULL) are divided by s[j], with the same rounding as
 * awq_fold_norm. W_prev must be 16-byte aligned with K_prev·element size a
 * multiple of 16 bytes; bias_prev aligned to its element size.
 * Does not synchronise. */
awq_status awq_fold_linear(void* W_prev, void* bias_prev, awq_dtype dtype, int64_t K,
                           int64_t K_prev, const float* s, void* stream);

/* Consumer of the packed layout (W4A16: 4-bit weights, 16-bit activations).
 * Y[t][n] = Σ_k X[t][k] · Ŵ[n][k] with Ŵ[n][k] = (q[k][n] - z[k/g][n]) ·
 * scale[k/g][n], reading qweight [K, N/8], qzeros [K/g, N/8] and scales
 * [K/g, N] (fp16 bits) exactly as awq_quantize_pack writes them at w_bit 4
 * ("05 — AWQ", section 5 "Bit-level output format"; the AWQ reading note,
 * "Key takeaways": weight-only INT4 inference with 16-bit activations).
 * X [T, K] holds the activations already divided by s (the fold), bf16 or
 * fp16; Y [T, N] is written in the same type. Ŵ is formed exactly in
 * float32; sums are float32, each output rounded once to nearest even.
 * T <= 16 runs a fused GEMV (Ŵ never stored). Larger T forms Ŵ rounded
 * once to the activation type for an MFMA GEMM, in one of two ways:
 *  - with ws_bytes >= awq_w4a16_workspace_bytes(T, N, K, dtype) (N·K 16-bit
 *    values), Ŵ is dequantised into the workspace first (the faster path);
 *  - with a smaller workspace (ws may then be NULL and ws_bytes 0) and
 *    K·N/2 < 2^31, the GEMM dequantises each k-tile on the fly and uses no
 *    workspace. Both give the same Y bit for bit.
 * N a multiple of 8, K of 128; group_size 32, 64 or 128. X and scales
 * 16-byte aligned, qweight and qzeros 4-byte, Y 2-byte, ws 16-byte.
 * A workspace too small for T <= 16, or for a layer the on-the-fly GEMM
 * cannot address: AWQ_E_WORKSPACE. Does not synchronise. */
size_t awq_w4a16_workspace_bytes(int64_t T, int64_t N, int64_t K, awq_dtype dtype);
awq_status awq_w4a16_matmul(const void* X, awq_dtype dtype, int64_t T, int64_t N, int64_t K,
                            const int32_t* qweight, const int32_t* qzeros,
                            const uint16_t* scales, int32_t group_size, void* Y, void* ws,
                            size_t ws_bytes, void* stream);

/* Message for the last non-OK status returned on the calling thread. */
const char* awq_last_error(void);

/* Kernel timing. When enabled, every kernel launch of the library is
 * bracketed by HIP events recorded on the stream it is launched on;
 * awq_profile_read synchronises those events and returns the summed
 * duration (ms) and launch count of one kernel kind since the last reset.
 * Kinds: 0 stats, 1 scale table, 2 transform (quantise/dequantise
 * candidates), 3 search GEMM, 4 reductions, 5 pack, 6 fold, 7 W4A16
 * dequantisation, 8 W4A16 GEMM or GEMV, 9 W4A16 GEMV reduction, 10 Gram
 * matrix build (transpose + G), 11 Gram-path candidate GEMM. */
enum { AWQ_K_STATS = 0, AWQ_K_SCALE = 1, AWQ_K_TRANSFORM = 2, AWQ_K_GEMM = 3, AWQ_K_REDUCE = 4,
       AWQ_K_PACK = 5, AWQ_K_FOLD = 6, AWQ_K_DEQUANT = 7, AWQ_K_W4A16 = 8,
       AWQ_K_W4A16_REDUCE = 9, AWQ_K_GRAM_BUILD = 10, AWQ_K_GRAM_SEARCH = 11, AWQ_K_COUNT = 12 };
void awq_profile_enable(int on);
void awq_profile_reset(void);
awq_status awq_profile_read(int kind, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* AWQ_MI355X_AWQ_H */
