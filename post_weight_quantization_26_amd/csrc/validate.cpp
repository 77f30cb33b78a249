// Argument checks and workspace arithmetic of the C ABI. Plain C++: no HIP
// headers and no HIP calls, so every rejection path runs on a machine
// without a GPU.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "awq_internal.h"

namespace awq {

static thread_local char g_err[512] = "";

awq_status set_error(awq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

static bool dtype_ok(awq_dtype d) { return d == AWQ_F32 || d == AWQ_BF16 || d == AWQ_F16; }

// Upper bound on any single dimension: fits an int, keeps every index
// product in int64.
static constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

int64_t stats_chunks(int64_t T, int64_t K, awq_dtype d) {
  const int64_t vec = 16 / int64_t(dtype_bytes(d));
  const int64_t col_blocks = ceil_div(K, 64 * vec);
  // at most 512 workgroups, 2 per CU (a third on some CUs left others idle
  // at the end: 11008 channels in 22 strips x 24 chunks ran 14% slower than
  // x 23), each with 4 loads in flight per lane: 32 KiB per CU in flight
  int64_t chunks = 512 / col_blocks;
  const int64_t max_chunks = ceil_div(T, 64);  // at least 64 rows (16 per row lane) per chunk
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks < 1) chunks = 1;
  return chunks;
}

int32_t gram_slices(int64_t T, int64_t K) {
  const int64_t Tp = ceil_div(T, kTileK) * kTileK;
  const int64_t nt = ceil_div(K, kGemmBM_bf16);
  const int64_t U = nt * (nt + 1) / 2;
  const int64_t ktiles = Tp / 64;
  int32_t best = 1;
  double best_cost = double(ceil_div(U, 256));
  for (int32_t S = 2; S <= 16 && 2 * S <= ktiles; ++S) {
    const double cost = double(ceil_div(U * S, 256)) / S;
    if (cost < best_cost) {
      best_cost = cost;
      best = S;
    }
  }
  return best;
}

GramBuildLayout gram_build_layout(int64_t T, int64_t K) {
  GramBuildLayout B{};
  B.Tp = ceil_div(T, kTileK) * kTileK;
  B.S = gram_slices(T, K);
  B.ldg = 2 * K + kGsPad;
  const size_t nt = size_t(ceil_div(K, kGemmBM_bf16));
  B.gp = 0;
  B.total = align_up(size_t(B.S) * (nt * (nt + 1) / 2) * 256 * 256 * 4);
  return B;
}

size_t gram_g_bytes(int64_t K) { return align_up(size_t(K) * size_t(2 * K + kGsPad) * 2); }

// The Gram search reads 256-row tiles of G's halves (rows of 2K + 256): they
// must fit the main loop's 32-bit tile offsets; the build's launch must fit
// the 32-bit grid. (The build reads X one 64-token k-tile at a time, so T
// needs no limit of its own.)
static awq_status check_gram_limits(const char* nm, int64_t T, int64_t K, bool build) {
  if (!tile_rows_fit(2 * K + kGsPad))
    return set_error(AWQ_E_UNSUPPORTED,
                     "%s: K=%lld exceeds the Gram search's 32-bit tile offsets "
                     "(512 * (2K + 256) must stay below 2^31)", nm, (long long)K);
  const int64_t nt = ceil_div(K, kGemmBM_bf16);
  // (the build's grid is its units rounded up to a multiple of 256)
  if (build && !grid_fits(ceil_div(nt * (nt + 1) / 2 * gram_slices(T, K), 256) * 256, 256))
    return set_error(AWQ_E_UNSUPPORTED, "%s: K=%lld exceeds the Gram build's grid", nm,
                     (long long)K);
  return AWQ_OK;
}

SearchLayout search_layout(int op, int64_t T, int64_t N, int64_t K, int32_t n_grid, int32_t nb,
                           awq_dtype dtype) {
  SearchLayout L{};
  const int64_t bm = dtype == AWQ_F32 ? kGemmBM_f32 : kGemmBM_bf16;
  const bool gram = is_gram_op(op), build = builds_gram(op);
  const GramBuildLayout B = build ? gram_build_layout(T, K) : GramBuildLayout{};
  L.MT = gram ? ceil_div(K, kGemmBM_bf16) : ceil_div(T, bm);
  L.Tp = B.Tp;
  L.S = B.S;
  L.ldg = gram ? 2 * K + kGsPad : 0;
  const size_t n_tab = is_scale_op(op) ? size_t(n_grid) : 1;
  size_t off = 0;
  L.s_table = off;
  off += align_up(n_tab * size_t(K) * 4);
  L.inv = off;
  off += align_up(n_tab * size_t(K) * 4);
  L.E = off;
  // fused searches: (step, zero, 1/step) per row and group of at least 32
  // channels, 16 bytes each
  off += align_up(is_fused_op(op) ? size_t(nb) * size_t(N) * size_t(K / 32) * 16
                                  : size_t(nb) * size_t(N) * size_t(K) * dtype_bytes(dtype) *
                                        (is_split_op(op) ? 2 : 1));
  L.partials = off;
  off += align_up(size_t(L.MT) * size_t(nb) * size_t(N) * 4);
  L.row_sums = off;
  off += align_up(size_t(n_grid) * size_t(N) * 8);
  L.mse = off;
  off += align_up(size_t(n_grid) * 8);
  L.best = off;
  off += align_up(size_t(N) * 8);
  L.scalar = off;
  off += align_up(64);
  // a building Gram search also holds the partial tiles and G
  L.gp = off + B.gp;
  off += B.total;
  L.gs = off;
  if (build) off += gram_g_bytes(K);
  L.total = off;
  return L;
}

awq_status check_gram_build(const void* X, awq_dtype d, int64_t T, int64_t K, const void* G,
                            size_t G_bytes, const void* ws, size_t ws_bytes) {
  if (!X || !G) return set_error(AWQ_E_INVALID, "gram_build: NULL X or G");
  if (!dtype_ok(d)) return set_error(AWQ_E_INVALID, "gram_build: unknown dtype %d", int(d));
  if (d != AWQ_BF16) return set_error(AWQ_E_UNSUPPORTED, "gram_build: bf16 inputs only");
  if (T < 1 || K < 1 || T > kMaxDim || K > kMaxDim)
    return set_error(AWQ_E_INVALID, "gram_build: bad shape T=%lld K=%lld", (long long)T,
                     (long long)K);
  if (K % kTileK)
    return set_error(AWQ_E_INVALID, "gram_build: K=%lld is not a multiple of 128", (long long)K);
  {
    awq_status st = check_gram_limits("gram_build", T, K, true);
    if (st != AWQ_OK) return st;
  }
  if (!aligned16(X) || !aligned16(G))
    return set_error(AWQ_E_INVALID, "gram_build: X and G must be 16-byte aligned");
  if (G_bytes < gram_g_bytes(K))
    return set_error(AWQ_E_WORKSPACE, "gram_build: G needs %zu bytes", gram_g_bytes(K));
  const size_t need = gram_build_layout(T, K).total;
  if (!ws || !aligned16(ws) || ws_bytes < need)
    return set_error(AWQ_E_WORKSPACE, "gram_build: workspace needs %zu bytes (16-byte aligned)",
                     need);
  return AWQ_OK;
}

awq_status check_stats_finalize(const double* sums, int64_t count, int64_t K, const float* abar) {
  if (!sums || !abar) return set_error(AWQ_E_INVALID, "act_stats_finalize: NULL sums or abar");
  if (count < 1 || K < 1 || K > kMaxDim)
    return set_error(AWQ_E_INVALID, "act_stats_finalize: bad count=%lld or K=%lld",
                     (long long)count, (long long)K);
  if ((reinterpret_cast<uintptr_t>(sums) & 7u) || !aligned4(abar))
    return set_error(AWQ_E_INVALID, "act_stats_finalize: sums must be 8-byte aligned, abar 4");
  return AWQ_OK;
}

awq_status check_stats_noalloc(const void* X, awq_dtype d, int64_t T, int64_t K,
                               const float* abar) {
  if (!X || !abar) return set_error(AWQ_E_INVALID, "act_stats_noalloc: NULL X or abar");
  if (!dtype_ok(d)) return set_error(AWQ_E_INVALID, "act_stats_noalloc: unknown dtype %d", int(d));
  if (T < 1 || K < 1 || T > kMaxDim || K > kMaxDim)
    return set_error(AWQ_E_INVALID, "act_stats_noalloc: bad shape T=%lld K=%lld", (long long)T,
                     (long long)K);
  const int64_t vec = 16 / int64_t(dtype_bytes(d));
  if (K % vec)
    return set_error(AWQ_E_INVALID, "act_stats_noalloc: K=%lld must be a multiple of %lld",
                     (long long)K, (long long)vec);
  if (!aligned16(X) || !aligned4(abar))
    return set_error(AWQ_E_INVALID, "act_stats_noalloc: X must be 16-byte aligned, abar 4");
  const int64_t need = stats_chunks(T, K, d) * K;
  if (need > kStatsScratchDoubles)
    return set_error(AWQ_E_UNSUPPORTED,
                     "act_stats_noalloc: %lld float64 partials exceed the static scratch of %lld "
                     "(use awq_act_stats with a workspace)",
                     (long long)need, (long long)kStatsScratchDoubles);
  return AWQ_OK;
}

awq_status check_stats(const void* X, awq_dtype d, int64_t T, int64_t K, const float* abar,
                       const void* ws, size_t ws_bytes) {
  if (!X || !abar) return set_error(AWQ_E_INVALID, "act_stats: NULL X or abar");
  if (!dtype_ok(d)) return set_error(AWQ_E_INVALID, "act_stats: unknown dtype %d", int(d));
  if (T < 1 || K < 1 || T > kMaxDim || K > kMaxDim)
    return set_error(AWQ_E_INVALID, "act_stats: bad shape T=%lld K=%lld", (long long)T,
                     (long long)K);
  const int64_t vec = 16 / int64_t(dtype_bytes(d));
  if (K % vec) return set_error(AWQ_E_INVALID, "act_stats: K=%lld must be a multiple of %lld",
                                (long long)K, (long long)vec);
  if (!aligned16(X) || !aligned4(abar))
    return set_error(AWQ_E_INVALID, "act_stats: X must be 16-byte aligned");
  const size_t need = awq_workspace_bytes(AWQ_OP_STATS, T, 1, K, 1, d);
  if (!ws || !aligned16(ws) || ws_bytes < need)
    return set_error(AWQ_E_WORKSPACE, "act_stats: workspace needs %zu bytes (16-byte aligned)",
                     need);
  return AWQ_OK;
}

awq_status check_scale_table(const float* abar, int64_t K, const float* alphas, int32_t n,
                             const float* s_table) {
  if (!abar || !alphas || !s_table) return set_error(AWQ_E_INVALID, "scale_table: NULL pointer");
  if (K < 1 || K > kMaxDim) return set_error(AWQ_E_INVALID, "scale_table: bad K");
  if (n < 1 || n > kMaxGrid)
    return set_error(AWQ_E_INVALID, "scale_table: n_alpha=%d outside 1..%d", n, kMaxGrid);
  for (int i = 0; i < n; ++i)
    if (!(alphas[i] >= 0.f && alphas[i] <= 1.f))
      return set_error(AWQ_E_INVALID, "scale_table: alpha[%d] outside [0, 1]", i);
  return AWQ_OK;
}

static awq_status check_qconfig(awq_qconfig qc) {
  if (qc.group_size != 32 && qc.group_size != 64 && qc.group_size != 128)
    return set_error(AWQ_E_UNSUPPORTED, "group_size %d not supported (32, 64 or 128)",
                     qc.group_size);
  if (qc.w_bit != 3 && qc.w_bit != 4)
    return set_error(AWQ_E_UNSUPPORTED, "w_bit %d not supported (3 or 4)", qc.w_bit);
  if (qc.zero_point != 0 && qc.zero_point != 1)
    return set_error(AWQ_E_INVALID, "zero_point must be 0 or 1");
  if (qc.flags != 0 && qc.flags != AWQ_SEARCH_SPLIT_E && qc.flags != AWQ_SEARCH_FUSED)
    return set_error(AWQ_E_INVALID, "flags must be 0, AWQ_SEARCH_SPLIT_E or AWQ_SEARCH_FUSED");
  return AWQ_OK;
}

awq_status check_search(int op, const void* X, const void* W, awq_dtype d, int64_t T, int64_t N,
                        int64_t K, const float* vec, const float* grid, int32_t n_grid,
                        awq_qconfig qc, const void* out_dev, const void* out_host,
                        const void* out_host2, const void* ws, size_t ws_bytes, int32_t* nb) {
  const char* nm = op == AWQ_OP_SEARCH_SCALE          ? "search_scale"
                   : op == AWQ_OP_SEARCH_CLIP         ? "search_clip"
                   : op == AWQ_OP_SEARCH_SCALE_GRAM   ? "search_scale_gram"
                   : op == AWQ_OP_SEARCH_CLIP_GRAM    ? "search_clip_gram"
                   : op == AWQ_OP_SEARCH_SCALE_GRAM_G ? "search_scale_gram_g"
                                                      : "search_clip_gram_g";
  // X is the prepared G for the _g searches
  if (!X || !W || !vec || !grid || !out_dev || !out_host || (is_scale_op(op) && !out_host2))
    return set_error(AWQ_E_INVALID, "%s: NULL pointer argument", nm);
  if (!dtype_ok(d)) return set_error(AWQ_E_INVALID, "%s: unknown dtype %d", nm, int(d));
  if (is_gram_op(op) && d != AWQ_BF16)
    return set_error(AWQ_E_UNSUPPORTED, "%s: the Gram path takes bf16 inputs", nm);
  if (is_gram_op(op) && (qc.flags & AWQ_SEARCH_SPLIT_E))
    return set_error(AWQ_E_UNSUPPORTED, "%s: split candidates are for the direct searches", nm);
  if ((qc.flags & AWQ_SEARCH_FUSED) && (is_gram_op(op) || d == AWQ_F32))
    return set_error(AWQ_E_UNSUPPORTED,
                     "%s: the fused search is for the direct searches of bf16 and fp16 layers", nm);
  if ((qc.flags & AWQ_SEARCH_FUSED) && N % 256)
    return set_error(AWQ_E_UNSUPPORTED, "%s: the fused search needs N a multiple of 256 (N=%lld)",
                     nm, (long long)N);
  if (T < 1 || N < 1 || K < 1 || T > kMaxDim || N > kMaxDim || K > kMaxDim)
    return set_error(AWQ_E_INVALID, "%s: bad shape T=%lld N=%lld K=%lld", nm, (long long)T,
                     (long long)N, (long long)K);
  awq_status st = check_qconfig(qc);
  if (st != AWQ_OK) return st;
  if (K % kTileK)
    return set_error(AWQ_E_INVALID, "%s: K=%lld is not a multiple of 128", nm, (long long)K);
  if (N * K > kMaxMatrixElems)
    return set_error(AWQ_E_UNSUPPORTED, "%s: N*K=%lld weights exceed 2^34 (32-bit grids)", nm,
                     (long long)(N * K));
  if (is_gram_op(op)) {
    st = check_gram_limits(nm, T, K, builds_gram(op));
    if (st != AWQ_OK) return st;
  } else if (d != AWQ_F32 && !tile_rows_fit(splits_e(qc, d) ? 2 * K : K)) {
    return set_error(AWQ_E_UNSUPPORTED,
                     "%s: K=%lld exceeds the search GEMM's 32-bit tile offsets (512 * K%s must "
                     "stay below 2^31)", nm, (long long)K, splits_e(qc, d) ? " * 2" : "");
  }
  if (n_grid < 1 || n_grid > kMaxGrid)
    return set_error(AWQ_E_INVALID, "%s: grid size %d outside 1..%d", nm, n_grid, kMaxGrid);
  for (int i = 0; i < n_grid; ++i) {
    const float g = grid[i];
    const bool ok = is_scale_op(op) ? (g >= 0.f && g <= 1.f) : (g > 0.f && g <= 1.f);
    if (!ok) return set_error(AWQ_E_INVALID, "%s: grid[%d]=%g out of range", nm, i, double(g));
  }
  if (!aligned16(X) || !aligned16(W) || !aligned4(vec) || !aligned4(out_dev))
    return set_error(AWQ_E_INVALID, "%s: X and W must be 16-byte aligned", nm);
  // the candidate GEMM of one batch covers b·N rows: its grid must fit
  auto blocks = [&](int32_t b) {
    return is_gram_op(op) ? gram_search_blocks(K, int64_t(b) * N)
                          : search_gemm_blocks(T, int64_t(b) * N, d);
  };
  if (!grid_fits(blocks(1), 256))
    return set_error(AWQ_E_UNSUPPORTED, "%s: T=%lld tokens x N=%lld rows exceed the 32-bit grid "
                     "of the candidate GEMM", nm, (long long)T, (long long)N);
  const int lop = layout_op(op, qc, d);
  const size_t need1 = search_layout(lop, T, N, K, n_grid, 1, d).total;
  if (!ws || !aligned16(ws) || ws_bytes < need1)
    return set_error(AWQ_E_WORKSPACE, "%s: workspace needs at least %zu bytes (16-byte aligned)",
                     nm, need1);
  int32_t b = n_grid;
  while (b > 1 && (search_layout(lop, T, N, K, n_grid, b, d).total > ws_bytes ||
                   !grid_fits(blocks(b), 256)))
    --b;
  *nb = b;
  return AWQ_OK;
}

awq_status check_group(const void* const* W, const int64_t* N, int32_t n_layers,
                       int64_t* N_total) {
  if (!W || !N) return set_error(AWQ_E_INVALID, "search_scale_group: NULL layer arrays");
  if (n_layers < 1 || n_layers > kMaxLayers)
    return set_error(AWQ_E_INVALID, "search_scale_group: n_layers=%d outside 1..%d", n_layers,
                     kMaxLayers);
  int64_t tot = 0;
  for (int l = 0; l < n_layers; ++l) {
    if (!W[l]) return set_error(AWQ_E_INVALID, "search_scale_group: W[%d] is NULL", l);
    if (!aligned16(W[l]))
      return set_error(AWQ_E_INVALID, "search_scale_group: W[%d] must be 16-byte aligned", l);
    if (N[l] < 1 || N[l] > kMaxDim)
      return set_error(AWQ_E_INVALID, "search_scale_group: N[%d]=%lld out of range", l,
                       (long long)N[l]);
    tot += N[l];
  }
  if (tot > kMaxDim)
    return set_error(AWQ_E_INVALID, "search_scale_group: %lld output channels in total",
                     (long long)tot);
  *N_total = tot;
  return AWQ_OK;
}

static bool aligned_elem(const void* p, awq_dtype d) {
  return d == AWQ_F32 ? aligned4(p) : (reinterpret_cast<uintptr_t>(p) & 1u) == 0;
}

awq_status check_fold_norm(const void* gamma, const void* beta, awq_dtype d, int64_t K,
                           const float* s) {
  if (!gamma || !s) return set_error(AWQ_E_INVALID, "fold_norm: NULL gamma or s");
  if (!dtype_ok(d)) return set_error(AWQ_E_INVALID, "fold_norm: unknown dtype %d", int(d));
  if (K < 1 || K > kMaxDim) return set_error(AWQ_E_INVALID, "fold_norm: bad K=%lld", (long long)K);
  if (!aligned_elem(gamma, d) || (beta && !aligned_elem(beta, d)) || !aligned4(s))
    return set_error(AWQ_E_INVALID, "fold_norm: misaligned pointer");
  return AWQ_OK;
}

awq_status check_fold_linear(const void* W_prev, const void* bias, awq_dtype d, int64_t K,
                             int64_t K_prev, const float* s) {
  if (!W_prev || !s) return set_error(AWQ_E_INVALID, "fold_linear: NULL W_prev or s");
  if (!dtype_ok(d)) return set_error(AWQ_E_INVALID, "fold_linear: unknown dtype %d", int(d));
  if (K < 1 || K_prev < 1 || K > kMaxDim || K_prev > kMaxDim)
    return set_error(AWQ_E_INVALID, "fold_linear: bad shape K=%lld K_prev=%lld", (long long)K,
                     (long long)K_prev);
  if (K * K_prev > kMaxMatrixElems)
    return set_error(AWQ_E_UNSUPPORTED, "fold_linear: K*K_prev=%lld elements exceed 2^34",
                     (long long)(K * K_prev));
  if ((K_prev * int64_t(dtype_bytes(d))) % 16)
    return set_error(AWQ_E_INVALID, "fold_linear: a row of W_prev (K_prev=%lld) must span a "
                     "multiple of 16 bytes", (long long)K_prev);
  if (!aligned16(W_prev) || (bias && !aligned_elem(bias, d)) || !aligned4(s))
    return set_error(AWQ_E_INVALID, "fold_linear: W_prev must be 16-byte aligned");
  return AWQ_OK;
}

awq_status check_pack(const void* W, awq_dtype d, int64_t N, int64_t K, const float* s,
                      awq_qconfig qc, const int32_t* qweight, const int32_t* qzeros,
                      const uint16_t* scales, const void* ws, size_t ws_bytes) {
  if (!W || !s || !qweight || !qzeros || !scales)
    return set_error(AWQ_E_INVALID, "quantize_pack: NULL pointer argument");
  if (!dtype_ok(d)) return set_error(AWQ_E_INVALID, "quantize_pack: unknown dtype %d", int(d));
  if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim)
    return set_error(AWQ_E_INVALID, "quantize_pack: bad shape N=%lld K=%lld", (long long)N,
                     (long long)K);
  awq_status st = check_qconfig(qc);
  if (st != AWQ_OK) return st;
  const int64_t n_mult = qc.w_bit == 4 ? 8 : 32;   // rows that fill whole 32-bit words
  if (N % n_mult)
    return set_error(AWQ_E_INVALID, "quantize_pack: N=%lld not a multiple of %lld for %d-bit codes",
                     (long long)N, (long long)n_mult, qc.w_bit);
  if (K % kTileK)
    return set_error(AWQ_E_INVALID, "quantize_pack: K=%lld not a multiple of 128", (long long)K);
  if (N * K > kMaxMatrixElems || !tile_rows_fit(K))
    return set_error(AWQ_E_UNSUPPORTED,
                     "quantize_pack: N*K=%lld weights exceed 2^34, or K=%lld its 32-bit tile "
                     "offsets (512 * K must stay below 2^31)", (long long)(N * K), (long long)K);
  if (N * 64 >= (int64_t(1) << 31))   // 128 qweight rows of N/8 words per workgroup
    return set_error(AWQ_E_UNSUPPORTED,
                     "quantize_pack: N=%lld exceeds the 32-bit offsets of a workgroup's qweight "
                     "rows (64 * N must stay below 2^31)", (long long)N);
  if (!aligned16(W) || !aligned4(qweight) || !aligned4(qzeros) || !aligned4(scales) ||
      !aligned4(s))
    return set_error(AWQ_E_INVALID, "quantize_pack: W must be 16-byte aligned, outputs 4-byte");
  const size_t need = awq_workspace_bytes(AWQ_OP_PACK, 1, N, K, 1, d);
  if (!ws || !aligned8(ws) || ws_bytes < need)
    return set_error(AWQ_E_WORKSPACE, "quantize_pack: workspace needs %zu bytes", need);
  return AWQ_OK;
}

int64_t w4a16_gemv_kpw(int64_t N, int64_t K) {
  const int64_t col_blocks = ceil_div(N / 8, 64);
  int64_t kpw = 128;
  while (kpw > 32 && (K % (4 * kpw) != 0 || col_blocks * (K / (4 * kpw)) < 1024)) kpw /= 2;
  return kpw;
}

// k rows per wave of the matrix-core GEMV: the largest of 512, 256, 128 that
// still gives 384 workgroups (1.5 per CU), else 128.
int64_t w4a16_mgemv_kpw(int64_t N, int64_t K) {
  const int64_t col_blocks = ceil_div(N / 8, 32);
  for (int64_t kpw = 512; kpw > 128; kpw /= 2)
    if (col_blocks * ceil_div(K, 4 * kpw) >= 384) return kpw;
  return 128;
}

awq_status check_w4a16(const void* X, awq_dtype d, int64_t T, int64_t N, int64_t K,
                       const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                       int32_t group, const void* Y, const void* ws, size_t ws_bytes) {
  if (!X || !qweight || !qzeros || !scales || !Y)
    return set_error(AWQ_E_INVALID, "w4a16_matmul: NULL pointer argument");
  if (!dtype_ok(d)) return set_error(AWQ_E_INVALID, "w4a16_matmul: unknown dtype %d", int(d));
  if (d == AWQ_F32)
    return set_error(AWQ_E_UNSUPPORTED, "w4a16_matmul: activations must be bf16 or fp16");
  if (T < 1 || N < 1 || K < 1 || T > kMaxDim || N > kMaxDim || K > kMaxDim)
    return set_error(AWQ_E_INVALID, "w4a16_matmul: bad shape T=%lld N=%lld K=%lld",
                     (long long)T, (long long)N, (long long)K);
  if (group != 32 && group != 64 && group != 128)
    return set_error(AWQ_E_UNSUPPORTED, "w4a16_matmul: group_size %d (32, 64 or 128)", group);
  if (N % 8) return set_error(AWQ_E_INVALID, "w4a16_matmul: N=%lld not a multiple of 8",
                              (long long)N);
  if (K % kTileK)
    return set_error(AWQ_E_INVALID, "w4a16_matmul: K=%lld not a multiple of 128", (long long)K);
  if (!tile_rows_fit(K) || N * K > kMaxMatrixElems)
    return set_error(AWQ_E_UNSUPPORTED,
                     "w4a16_matmul: K=%lld, N=%lld exceed the 32-bit offsets (512 * K must stay "
                     "below 2^31, N*K at most 2^34)", (long long)K, (long long)N);
  if (T > kW4A16GemvMaxT && !grid_fits(search_gemm_blocks(T, N, AWQ_BF16), 256))
    return set_error(AWQ_E_UNSUPPORTED, "w4a16_matmul: T=%lld x N=%lld exceed the GEMM's grid",
                     (long long)T, (long long)N);
  if (!aligned16(X) || !aligned4(qweight) || !aligned4(qzeros) || !aligned16(scales) ||
      (reinterpret_cast<uintptr_t>(Y) & 1u))
    return set_error(AWQ_E_INVALID,
                     "w4a16_matmul: X and scales must be 16-byte aligned, qweight/qzeros 4, Y 2");
  const size_t need = awq_w4a16_workspace_bytes(T, N, K, d);
  // prefill with a smaller workspace (or none): the GEMM dequantises on the fly
  if (T > kW4A16GemvMaxT && ws_bytes < need && w4a16_fused_fits(N, K)) return AWQ_OK;
  if (!ws || !aligned16(ws) || ws_bytes < need)
    return set_error(AWQ_E_WORKSPACE, "w4a16_matmul: workspace needs %zu bytes (16-byte aligned)",
                     need);
  return AWQ_OK;
}


awq_status check_w3a16(const void* X, awq_dtype d, int64_t T, int64_t N, int64_t K,
                       const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                       int32_t group, const void* Y, const void* ws, size_t ws_bytes) {
  if (!X || !qweight || !qzeros || !scales || !Y)
    return set_error(AWQ_E_INVALID, "w3a16_matmul: NULL pointer argument");
  if (!dtype_ok(d)) return set_error(AWQ_E_INVALID, "w3a16_matmul: unknown dtype %d", int(d));
  if (d == AWQ_F32)
    return set_error(AWQ_E_UNSUPPORTED, "w3a16_matmul: activations must be bf16 or fp16");
  if (T < 1 || N < 1 || K < 1 || T > kMaxDim || N > kMaxDim || K > kMaxDim)
    return set_error(AWQ_E_INVALID, "w3a16_matmul: bad shape T=%lld N=%lld K=%lld",
                     (long long)T, (long long)N, (long long)K);
  if (group != 32 && group != 64 && group != 128)
    return set_error(AWQ_E_UNSUPPORTED, "w3a16_matmul: group_size %d (32, 64 or 128)", group);
  if (N % 32) return set_error(AWQ_E_INVALID, "w3a16_matmul: N=%lld not a multiple of 32",
                               (long long)N);
  if (K % kTileK)
    return set_error(AWQ_E_INVALID, "w3a16_matmul: K=%lld not a multiple of 128", (long long)K);
  if (!tile_rows_fit(K) || N * K > kMaxMatrixElems)
    return set_error(AWQ_E_UNSUPPORTED,
                     "w3a16_matmul: K=%lld, N=%lld exceed the 32-bit offsets (512 * K must stay "
                     "below 2^31, N*K at most 2^34)", (long long)K, (long long)N);
  if (T > kW4A16GemvMaxT && !grid_fits(search_gemm_blocks(T, N, AWQ_BF16), 256))
    return set_error(AWQ_E_UNSUPPORTED, "w3a16_matmul: T=%lld x N=%lld exceed the GEMM's grid",
                     (long long)T, (long long)N);
  if (!aligned16(X) || !aligned4(qweight) || !aligned4(qzeros) || !aligned16(scales) ||
      (reinterpret_cast<uintptr_t>(Y) & 1u))
    return set_error(AWQ_E_INVALID,
                     "w3a16_matmul: X and scales must be 16-byte aligned, qweight/qzeros 4, Y 2");
  const size_t need = awq_w3a16_workspace_bytes(T, N, K, d);
  if (!ws || !aligned16(ws) || ws_bytes < need)
    return set_error(AWQ_E_WORKSPACE, "w3a16_matmul: workspace needs %zu bytes (16-byte aligned)",
                     need);
  return AWQ_OK;
}

}  // namespace awq

extern "C" size_t awq_w4a16_workspace_bytes(int64_t T, int64_t N, int64_t K, awq_dtype dtype) {
  using namespace awq;
  if (T < 1 || N < 1 || K < 1 || T > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  if (dtype != AWQ_BF16 && dtype != AWQ_F16) return 0;
  if (N % 8 || K % kTileK) return 0;
  if (T <= kW4A16GemvMaxT) {
    // either decode path, whichever the pointers select
    const int64_t chunks = N % 16 ? w4a16_gemv_chunks(N, K)
                                  : std::max(w4a16_gemv_chunks(N, K), w4a16_mgemv_chunks(N, K));
    return align_up(size_t(chunks) * size_t(T) * size_t(N) * 4);
  }
  return align_up(size_t(N) * size_t(K) * 2);
}

extern "C" size_t awq_w3a16_workspace_bytes(int64_t T, int64_t N, int64_t K, awq_dtype dtype) {
  using namespace awq;
  if (T < 1 || N < 1 || K < 1 || T > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  if (dtype != AWQ_BF16 && dtype != AWQ_F16) return 0;
  if (N % 32 || K % kTileK) return 0;
  if (T <= kW4A16GemvMaxT)
    return align_up(size_t(w4a16_mgemv_chunks(N, K)) * size_t(T) * size_t(N) * 4);
  return align_up(size_t(N) * size_t(K) * 2);
}

extern "C" size_t awq_workspace_bytes(int op, int64_t T, int64_t N, int64_t K, int32_t n_grid,
                                      awq_dtype dtype) {
  using namespace awq;
  if (T < 1 || N < 1 || K < 1 || n_grid < 1 || n_grid > kMaxGrid) return 0;
  if (T > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  if (!(dtype == AWQ_F32 || dtype == AWQ_BF16 || dtype == AWQ_F16)) return 0;
  switch (op) {
    case AWQ_OP_STATS:
      return align_up(size_t(stats_chunks(T, K, dtype)) * size_t(K) * 8);
    case AWQ_OP_SEARCH_SCALE:
    case AWQ_OP_SEARCH_CLIP:
      return search_layout(op, T, N, K, n_grid, n_grid, dtype).total;
    case AWQ_OP_SEARCH_SCALE_SPLIT_E:
    case AWQ_OP_SEARCH_CLIP_SPLIT_E:
      // float32 layers do not split: their searches use the plain layout
      return search_layout(dtype == AWQ_F32 ? unsplit_op(op) : op, T, N, K, n_grid, n_grid,
                           dtype).total;
    case AWQ_OP_SEARCH_SCALE_FUSED:
    case AWQ_OP_SEARCH_CLIP_FUSED:
      if (dtype == AWQ_F32 || K % kTileK) return 0;   // 16-bit layers only
      return search_layout(op, T, N, K, n_grid, n_grid, dtype).total;
    case AWQ_OP_SEARCH_SCALE_GRAM:
    case AWQ_OP_SEARCH_CLIP_GRAM:
    case AWQ_OP_SEARCH_SCALE_GRAM_G:
    case AWQ_OP_SEARCH_CLIP_GRAM_G:
      if (dtype != AWQ_BF16 || K % kTileK) return 0;
      return search_layout(op, T, N, K, n_grid, n_grid, dtype).total;
    case AWQ_OP_GRAM_BUILD:
      if (dtype != AWQ_BF16 || K % kTileK) return 0;
      return gram_build_layout(T, K).total;
    case AWQ_OP_PACK:
      return kAlign;
    default:
      return 0;
  }
}

extern "C" size_t awq_workspace_bytes_batch(int op, int64_t T, int64_t N, int64_t K,
                                            int32_t n_grid, int32_t batch, awq_dtype dtype) {
  using namespace awq;
  if (op != AWQ_OP_SEARCH_SCALE && op != AWQ_OP_SEARCH_CLIP && !is_gram_op(op) &&
      !is_split_op(op) && !is_fused_op(op))
    return 0;
  if (batch < 1 || batch > n_grid) return 0;
  if (awq_workspace_bytes(op, T, N, K, n_grid, dtype) == 0) return 0;
  if (dtype == AWQ_F32) op = unsplit_op(op);   // float32 layers do not split
  return search_layout(op, T, N, K, n_grid, batch, dtype).total;
}

extern "C" size_t awq_gram_bytes(int64_t K) {
  using namespace awq;
  if (K < 1 || K > kMaxDim || K % kTileK) return 0;
  return gram_g_bytes(K);
}

extern "C" const char* awq_last_error(void) { return awq::g_err; }
