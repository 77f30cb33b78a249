// Internal declarations shared by the C ABI and the HIP kernels. Host-only
// types: nothing here needs the HIP headers, so the argument checks and the
// workspace arithmetic can be compiled and tested without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

#include "awq.h"

namespace awq {

constexpr int kTileK = 128;   // K must be a multiple of this (search GEMM and pack tiles)
constexpr int kMaxGrid = 64;
constexpr int kMaxLayers = 16;     // linears searched together on one shared input
constexpr int kGemmBM_bf16 = 256;  // token rows per search-GEMM tile (bf16 MFMA path)
constexpr int kGemmBM_f32 = 64;    // token rows per tile on the fp32 path
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t dtype_bytes(awq_dtype d) { return d == AWQ_F32 ? 4 : 2; }

// Addressing limits of the kernels, checked on the host before any launch.
//  * The MFMA main loop reads a 256-row tile of a 16-bit operand through a
//    buffer resource with 32-bit byte offsets and size: 256 rows times the
//    row length times 2 bytes must stay below 2^31.
//  * A launch holds fewer than 2^32 work-items (grids are 32-bit); the
//    widest element-wise launches (candidate transform, pack, dequantise,
//    fold) take 8 elements per lane, so their matrices hold at most 2^34
//    elements.
constexpr int64_t kMaxMatrixElems = int64_t(1) << 34;
inline bool tile_rows_fit(int64_t row_elems) {
  return row_elems >= 0 && row_elems < (int64_t(1) << 22);
}
inline bool grid_fits(int64_t blocks, int64_t threads_per_block) {
  return blocks >= 0 && blocks * threads_per_block < (int64_t(1) << 32);
}
// Workgroups of the search GEMM for T token rows and Nc candidate rows
// (16-bit: 256 x 256 tiles, XCD-grouped; float32: 64 x 64 tiles), and of the
// Gram search for K channels and Nc candidate rows. 256 threads each.
inline int64_t search_gemm_blocks(int64_t T, int64_t Nc, awq_dtype d) {
  if (d == AWQ_F32) return ceil_div(T, 64) * ceil_div(Nc, 64);
  const int64_t tm = ceil_div(T, 256), tn = ceil_div(Nc, 256);
  if (tm >= 32) return ceil_div(tm, 32) * 32 * (ceil_div(tn, 8) * 8);
  if (tm == 16 || tm == 8 || tm == 4) return ceil_div(tn, 64 / (tm / 4)) * 256;
  return tm * tn;
}
inline int64_t gram_search_blocks(int64_t K, int64_t Nc) {
  return ceil_div(ceil_div(K, 256), 2) * 8 * ceil_div(ceil_div(Nc, 256), 8);
}

// Number of token chunks the stats kernel splits T into (one float64 partial
// row per chunk); chosen so the launch has at most 512 workgroups, 2 per CU.
int64_t stats_chunks(int64_t T, int64_t K, awq_dtype d);

// Byte offsets of the regions of a search workspace for a batch of `nb`
// candidates out of `n_grid`.
struct SearchLayout {
  size_t s_table;   // [n_grid, K] f32 scale table (clip search: aligned copy of s, [K])
  size_t inv;       // [n_grid, K] f32 reciprocal scales (clip search: [K])
  size_t E;         // [nb, N, K] candidate error weights (bf16, fp16 or f32; split: [nb, N, 2K])
  size_t partials;  // [MT, nb*N] f32 per-tile column sums of squares
  size_t row_sums;  // [n_grid, N] f64
  size_t mse;       // [n_grid] f64
  size_t best;      // [N] f64 best per-row sums (clip search)
  size_t scalar;    // [8] f64
  size_t gp;        // Gram searches: [S, U, 256, 256] f32 partial tiles of G
  size_t gs;        // Gram searches: [K, 2K + 256] bf16, G's upper tiles as hi/lo halves
  size_t total;
  int64_t MT;       // row tiles of the partials (token tiles; Gram: channel tiles)
  int64_t Tp;       // Gram searches: tokens padded to a multiple of 128
  int64_t ldg;      // Gram searches: row stride of Gs in elements (>= 2K)
  int32_t S;        // Gram searches: token slices of the G build
};

// Row padding of Gs (elements). Unpadded, its row stride is a power of two
// at typical sizes (32 KiB at K = 8192), so the 256 rows of one k-tile fall
// on few cache sets and memory channels. Measured: 256 more elements per row
// cut the K = 8192 search by ~8% (neutral at K = 4096).
constexpr int64_t kGsPad = 256;

// Token slices of the Gram build: the S <= 16 (slices of at least two
// 64-token k-tiles, lengths differing by at most one k-tile) that finishes
// the U·S (upper tile, slice) units of work in the fewest rounds of 256 CUs
// relative to the slice length (ties to the smaller S).
int32_t gram_slices(int64_t T, int64_t K);

// Gram searches: those that build G in their own workspace, and those that
// read a prepared G.
inline bool builds_gram(int op) {
  return op == AWQ_OP_SEARCH_SCALE_GRAM || op == AWQ_OP_SEARCH_CLIP_GRAM;
}
inline bool is_gram_op(int op) {
  return builds_gram(op) || op == AWQ_OP_SEARCH_SCALE_GRAM_G || op == AWQ_OP_SEARCH_CLIP_GRAM_G;
}
inline bool is_scale_op(int op) {
  return op == AWQ_OP_SEARCH_SCALE || op == AWQ_OP_SEARCH_SCALE_GRAM ||
         op == AWQ_OP_SEARCH_SCALE_GRAM_G || op == AWQ_OP_SEARCH_SCALE_SPLIT_E ||
         op == AWQ_OP_SEARCH_SCALE_FUSED;
}
// Direct searches that form the candidates in the search GEMM: their
// candidate region holds float4 group parameters, at most K/2 bytes a row.
inline bool is_fused_op(int op) {
  return op == AWQ_OP_SEARCH_SCALE_FUSED || op == AWQ_OP_SEARCH_CLIP_FUSED;
}
// Direct searches whose candidates are hi/lo halves (rows of 2K elements).
inline bool is_split_op(int op) {
  return op == AWQ_OP_SEARCH_SCALE_SPLIT_E || op == AWQ_OP_SEARCH_CLIP_SPLIT_E;
}
inline int unsplit_op(int op) {
  return op == AWQ_OP_SEARCH_SCALE_SPLIT_E ? AWQ_OP_SEARCH_SCALE
         : op == AWQ_OP_SEARCH_CLIP_SPLIT_E ? AWQ_OP_SEARCH_CLIP
                                            : op;
}
// The search splits the candidates' error weights: asked for, on a 16-bit
// layer (float32 layers keep float32 operands).
inline bool splits_e(awq_qconfig qc, awq_dtype d) {
  return (qc.flags & AWQ_SEARCH_SPLIT_E) && d != AWQ_F32;
}
// The op whose workspace layout a search call uses: its split or fused form
// when the call splits or fuses its candidates.
inline int layout_op(int op, awq_qconfig qc, awq_dtype d) {
  if ((qc.flags & AWQ_SEARCH_FUSED) && d != AWQ_F32) {
    if (op == AWQ_OP_SEARCH_SCALE) return AWQ_OP_SEARCH_SCALE_FUSED;
    if (op == AWQ_OP_SEARCH_CLIP) return AWQ_OP_SEARCH_CLIP_FUSED;
    return op;
  }
  if (!splits_e(qc, d)) return op;
  if (op == AWQ_OP_SEARCH_SCALE) return AWQ_OP_SEARCH_SCALE_SPLIT_E;
  if (op == AWQ_OP_SEARCH_CLIP) return AWQ_OP_SEARCH_CLIP_SPLIT_E;
  return op;
}
// The partial tiles of a G build (the first part of a building Gram search's
// workspace, and the whole workspace of awq_gram_build).
struct GramBuildLayout {
  int64_t Tp, ldg;
  int32_t S;
  size_t gp, total;
};
GramBuildLayout gram_build_layout(int64_t T, int64_t K);
size_t gram_g_bytes(int64_t K);
awq_status check_gram_build(const void* X, awq_dtype d, int64_t T, int64_t K, const void* G,
                            size_t G_bytes, const void* ws, size_t ws_bytes);
SearchLayout search_layout(int op, int64_t T, int64_t N, int64_t K, int32_t n_grid, int32_t nb,
                           awq_dtype dtype);

// Host-side argument checks. Return AWQ_OK or an error (message via set_error).
awq_status check_stats_finalize(const double* sums, int64_t count, int64_t K, const float* abar);
awq_status check_stats(const void* X, awq_dtype d, int64_t T, int64_t K, const float* abar,
                       const void* ws, size_t ws_bytes);
// awq_act_stats_noalloc: the float64 chunk partials live in a static device
// array of this many doubles (8 MiB per device); larger calls are refused.
constexpr int64_t kStatsScratchDoubles = int64_t(1) << 20;
awq_status check_stats_noalloc(const void* X, awq_dtype d, int64_t T, int64_t K,
                               const float* abar);
awq_status check_scale_table(const float* abar, int64_t K, const float* alphas, int32_t n,
                             const float* s_table);
awq_status check_search(int op, const void* X, const void* W, awq_dtype d, int64_t T, int64_t N,
                        int64_t K, const float* vec, const float* grid, int32_t n_grid,
                        awq_qconfig qc, const void* out_dev, const void* out_host,
                        const void* out_host2, const void* ws, size_t ws_bytes, int32_t* nb);
// Layers of a shared-input group: non-NULL 16-byte aligned weights, sizes
// >= 1; *N_total receives the summed output channels.
awq_status check_group(const void* const* W, const int64_t* N, int32_t n_layers, int64_t* N_total);
awq_status check_fold_norm(const void* gamma, const void* beta, awq_dtype d, int64_t K,
                           const float* s);
awq_status check_fold_linear(const void* W_prev, const void* bias, awq_dtype d, int64_t K,
                             int64_t K_prev, const float* s);
awq_status check_pack(const void* W, awq_dtype d, int64_t N, int64_t K, const float* s,
                      awq_qconfig qc, const int32_t* qweight, const int32_t* qzeros,
                      const uint16_t* scales, const void* ws, size_t ws_bytes);

// W4A16 consumer: token rows up to which the fused GEMV path runs; rows of k
// per wave of the GEMV (the largest of 128, 64, 32 dividing K/4 that still
// gives >= 1024 workgroups); its number of k chunks.
constexpr int64_t kW4A16GemvMaxT = 16;
int64_t w4a16_gemv_kpw(int64_t N, int64_t K);
inline int64_t w4a16_gemv_chunks(int64_t N, int64_t K) { return K / (4 * w4a16_gemv_kpw(N, K)); }
// Decode on the matrix cores: N a multiple of 16 and qweight/qzeros 8-byte
// aligned (a lane reads two adjacent word columns at once); otherwise the
// float32 GEMV above.
inline bool w4a16_use_mgemv(int64_t N, const void* qweight, const void* qzeros) {
  return N % 16 == 0 && (reinterpret_cast<uintptr_t>(qweight) & 7u) == 0 &&
         (reinterpret_cast<uintptr_t>(qzeros) & 7u) == 0;
}
// The prefill GEMM that dequantises on the fly addresses qweight with 32-bit
// buffer offsets: K·N/2 < 2^31 bytes.
inline bool w4a16_fused_fits(int64_t N, int64_t K) {
  return K * (N / 8) * 4 < (int64_t(1) << 31);
}
int64_t w4a16_mgemv_kpw(int64_t N, int64_t K);
inline int64_t w4a16_mgemv_chunks(int64_t N, int64_t K) {
  const int64_t span = 4 * w4a16_mgemv_kpw(N, K);
  return (K + span - 1) / span;
}
awq_status check_w3a16(const void* X, awq_dtype d, int64_t T, int64_t N, int64_t K,
                       const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                       int32_t group, const void* Y, const void* ws, size_t ws_bytes);
awq_status check_w4a16(const void* X, awq_dtype d, int64_t T, int64_t N, int64_t K,
                       const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                       int32_t group, const void* Y, const void* ws, size_t ws_bytes);

awq_status set_error(awq_status st, const char* fmt, ...);

}  // namespace awq
