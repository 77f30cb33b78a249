// The C ABI entry points: validate on the host, then enqueue the HIP kernels
// on the caller's stream. See include/awq.h for the contract of each call.
#include <cmath>
#include <hip/hip_runtime_api.h>

#include <cstring>
#include <mutex>
#include <vector>

#include "awq_internal.h"

namespace awq {
// Launchers (HIP translation units).
hipError_t launch_stats(const void* X, int dtype, int64_t T, int64_t K, int64_t chunks,
                        double* partial, float* abar, hipStream_t st);
hipError_t stats_scratch(double** out);
hipError_t launch_scale_table(const float* abar, int64_t K, const float* alphas_host, int n,
                              float* s_table, float* inv_table, hipStream_t st);
hipError_t launch_reciprocal(const float* s, int64_t n, float* s_copy, float* inv,
                             hipStream_t st);
hipError_t launch_transform(const void* W, int dtype, int64_t N, int64_t K, const float* s_rows,
                            const float* inv_rows, int64_t s_stride, const float* ratios_host,
                            int nc, int bits, int group, int zero_point, int split, void* E,
                            int64_t cand_stride, hipStream_t st);
hipError_t launch_search_gemm(const void* X, int dtype, const void* E, int64_t M, int64_t Nc,
                              int64_t K, int split, float* partials, hipStream_t st);
hipError_t launch_group_params(const void* W, int dtype, int64_t N, int64_t K,
                               const float* s_rows, int64_t s_stride, const float* ratios_host,
                               int nc, int bits, int group, int zero_point, float* P,
                               int64_t cand_stride, hipStream_t st);
hipError_t launch_search_fused(const void* X, int dtype, const void* W, const float* P,
                               const float* s_rows, const float* inv_rows, int64_t s_stride,
                               int64_t M, int64_t N, int64_t K, int nc, int group, int bits,
                               float* partials, hipStream_t st);
hipError_t launch_reduce_rows(const float* partials, int64_t MT, int64_t Nc, double* row_sums,
                              hipStream_t st);
hipError_t launch_curve(const double* row_sums, int n_cand, int64_t N, double denom,
                        double* mse, hipStream_t st);
hipError_t launch_clip_select(const double* row_sums, int n_ratio, int64_t N,
                              const float* ratios_host, double denom, float* ratio_best,
                              double* best, double* mse_clip, hipStream_t st);
hipError_t launch_pack(const void* W, int dtype, int64_t N, int64_t K, const float* s,
                       const float* ratio, int bits, int group, int zero_point, int32_t* qweight,
                       int32_t* qzeros, uint16_t* scales, int* overflow, hipStream_t st);
hipError_t launch_w4a16_dequant(const int32_t* qweight, const int32_t* qzeros,
                                const uint16_t* scales, int64_t N, int64_t K, int group, int f16,
                                uint16_t* Wd, hipStream_t st);
hipError_t launch_w3a16_dequant(const int32_t* qweight, const int32_t* qzeros,
                                const uint16_t* scales, int64_t N, int64_t K, int group, int f16,
                                uint16_t* Wd, hipStream_t st);
hipError_t launch_w4a16_gemm(const uint16_t* X, const uint16_t* Wd, int64_t M, int64_t N,
                             int64_t K, int f16, uint16_t* Y, hipStream_t st);
hipError_t launch_w4a16_gemv(const uint16_t* X, int64_t T, int64_t N, int64_t K,
                             const int32_t* qweight, const int32_t* qzeros,
                             const uint16_t* scales, int group, int f16, int64_t kpw,
                             float* partial, hipStream_t st);
hipError_t launch_w4a16_mgemv(const uint16_t* X, int64_t T, int64_t N, int64_t K,
                              const int32_t* qweight, const int32_t* qzeros,
                              const uint16_t* scales, int group, int f16, int64_t kpw,
                              float* partial, hipStream_t st, int bits);
hipError_t launch_w4a16_gemm_q(const uint16_t* X, const int32_t* qweight, const int32_t* qzeros,
                               const uint16_t* scales, int64_t M, int64_t N, int64_t K,
                               int group, int f16, uint16_t* Y, hipStream_t st);
hipError_t launch_w4a16_gemv_reduce(const float* partial, int64_t chunks, int64_t T, int64_t N,
                                    int f16, uint16_t* Y, hipStream_t st);
hipError_t launch_stats_accumulate(const void* X, int dtype, int64_t T, int64_t K,
                                   int64_t chunks, double* partial, double* sums, hipStream_t st);
hipError_t launch_stats_divide(const double* sums, int64_t count, int64_t K, float* abar,
                               hipStream_t st);
hipError_t launch_gram_build(const void* X, int64_t T, int64_t K, int64_t Tp, int S, float* P,
                             int64_t ldg, uint16_t* Gs, hipStream_t st);
hipError_t launch_gram_search(const uint16_t* Gs, int64_t ldg, const void* E, int64_t K, int64_t Nc,
                              float* partials, hipStream_t st);
hipError_t launch_fold_vec(void* v, int dtype, int64_t K, const float* s, hipStream_t st);
hipError_t launch_fold_rows(void* W, int dtype, int64_t K, int64_t K_prev, const float* s,
                            hipStream_t st);

namespace {

// ---------------------------------------------------------------------------
// Optional kernel timing with HIP events on the launch stream.
// ---------------------------------------------------------------------------
struct Pending {
  int kind;
  hipEvent_t a, b;
};

struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<Pending> pending;
  std::vector<hipEvent_t> spare;
  double ms[AWQ_K_COUNT] = {};
  int64_t n[AWQ_K_COUNT] = {};
};

Profiler& prof() {
  static Profiler p;
  return p;
}

hipEvent_t take_event() {
  Profiler& p = prof();
  if (!p.spare.empty()) {
    hipEvent_t e = p.spare.back();
    p.spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <class F>
hipError_t timed(int kind, hipStream_t st, F&& launch) {
  Profiler& p = prof();
  std::unique_lock<std::mutex> lk(p.mu);
  if (!p.on) {
    lk.unlock();
    return launch();
  }
  // a timing is kept only when both events were created and recorded; the
  // launch's own status is what the caller sees either way
  hipEvent_t a = take_event(), b = take_event();
  const bool started = a && b && hipEventRecord(a, st) == hipSuccess;
  hipError_t e = launch();
  if (started && hipEventRecord(b, st) == hipSuccess) {
    p.pending.push_back({kind, a, b});
  } else {
    if (a) p.spare.push_back(a);
    if (b) p.spare.push_back(b);
  }
  return e;
}

awq_status hip_fail(hipError_t e, const char* where) {
  return set_error(AWQ_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define AWQ_HIP(call, where)                     \
  do {                                           \
    hipError_t e__ = (call);                     \
    if (e__ != hipSuccess) return hip_fail(e__, where); \
  } while (0)

int dt(awq_dtype d) { return d == AWQ_F32 ? 0 : d == AWQ_BF16 ? 1 : 2; }

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// One layer of a search: its weights and its first row among the N output
// channels searched together.
struct Segment {
  const void* W;
  int64_t N;
  int64_t row0;
};

// Runs transform -> GEMM -> row reduction for candidates [c0, c0+cb). E holds
// candidate blocks of N rows each; every segment fills its rows of every block.
// With Gs (the Gram halves of G) the candidate GEMM is E·G·Eᵀ per row instead
// of the direct X·Eᵀ.
awq_status run_batch(const void* X, const Segment* seg, int n_seg, awq_dtype d, int64_t T,
                     int64_t N, int64_t K, const float* s_rows, const float* inv_rows,
                     int64_t s_stride, const float* ratios_host, int cb, awq_qconfig qc,
                     const SearchLayout& L, void* ws, double* row_sums_out, hipStream_t st,
                     const uint16_t* Gs = nullptr) {
  void* E = at<void>(ws, L.E);
  float* partials = at<float>(ws, L.partials);
  if (qc.flags & AWQ_SEARCH_FUSED) {
    // one layer (checked): its group parameters go where E would, and the
    // search GEMM forms the candidates from W
    float* P = static_cast<float*>(E);
    const int64_t pstride = N * (K / qc.group_size);
    AWQ_HIP(timed(AWQ_K_TRANSFORM, st,
                  [&] {
                    return launch_group_params(seg[0].W, dt(d), N, K, s_rows, s_stride,
                                               ratios_host, cb, qc.w_bit, qc.group_size,
                                               qc.zero_point, P, pstride, st);
                  }),
            "group_params");
    AWQ_HIP(timed(AWQ_K_GEMM, st,
                  [&] {
                    return launch_search_fused(X, dt(d), seg[0].W, P, s_rows, inv_rows, s_stride,
                                               T, N, K, cb, qc.group_size, qc.w_bit, partials,
                                               st);
                  }),
            "search_fused");
    AWQ_HIP(timed(AWQ_K_REDUCE, st,
                  [&] {
                    return launch_reduce_rows(partials, L.MT, int64_t(cb) * N, row_sums_out, st);
                  }),
            "reduce_rows");
    return AWQ_OK;
  }
  // split candidates: each row is a hi and a lo half (2K elements)
  const int split = splits_e(qc, d);
  const int64_t row_len = split ? 2 * K : K;
  for (int l = 0; l < n_seg; ++l) {
    void* E_l = static_cast<char*>(E) + size_t(seg[l].row0) * size_t(row_len) * dtype_bytes(d);
    AWQ_HIP(timed(AWQ_K_TRANSFORM, st,
                  [&] {
                    return launch_transform(seg[l].W, dt(d), seg[l].N, K, s_rows, inv_rows,
                                            s_stride, ratios_host, cb, qc.w_bit, qc.group_size,
                                            qc.zero_point, split, E_l, N * row_len, st);
                  }),
            "transform");
  }
  if (Gs)
    AWQ_HIP(timed(AWQ_K_GRAM_SEARCH, st,
                  [&] { return launch_gram_search(Gs, L.ldg, E, K, int64_t(cb) * N, partials, st); }),
            "gram_search");
  else
    AWQ_HIP(timed(AWQ_K_GEMM, st,
                  [&] {
                    return launch_search_gemm(X, dt(d), E, T, int64_t(cb) * N, K, split,
                                              partials, st);
                  }),
            "search_gemm");
  AWQ_HIP(timed(AWQ_K_REDUCE, st,
                [&] { return launch_reduce_rows(partials, L.MT, int64_t(cb) * N, row_sums_out, st); }),
          "reduce_rows");
  return AWQ_OK;
}

}  // namespace
}  // namespace awq

using namespace awq;

extern "C" awq_status awq_act_stats(const void* X, awq_dtype x_dtype, int64_t T, int64_t K,
                                    float* abar, void* ws, size_t ws_bytes, void* stream) {
  awq_status s = check_stats(X, x_dtype, T, K, abar, ws, ws_bytes);
  if (s != AWQ_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t chunks = stats_chunks(T, K, x_dtype);
  AWQ_HIP(timed(AWQ_K_STATS, st,
                [&] {
                  return launch_stats(X, dt(x_dtype), T, K, chunks, static_cast<double*>(ws), abar,
                                      st);
                }),
          "act_stats");
  return AWQ_OK;
}

extern "C" awq_status awq_act_stats_noalloc(const void* X, awq_dtype x_dtype, int64_t T,
                                            int64_t K, float* abar, void* stream) {
  awq_status s = check_stats_noalloc(X, x_dtype, T, K, abar);
  if (s != AWQ_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  double* partial = nullptr;
  AWQ_HIP(stats_scratch(&partial), "act_stats_noalloc: scratch address");
  // the same kernels as awq_act_stats with the static scratch as their
  // workspace; no profiler events (they would be created on first use)
  AWQ_HIP(launch_stats(X, dt(x_dtype), T, K, stats_chunks(T, K, x_dtype), partial, abar, st),
          "act_stats_noalloc");
  return AWQ_OK;
}

extern "C" awq_status awq_act_stats_accumulate(const void* X, awq_dtype x_dtype, int64_t T,
                                               int64_t K, double* sums, void* ws,
                                               size_t ws_bytes, void* stream) {
  if (!sums) return set_error(AWQ_E_INVALID, "act_stats_accumulate: NULL sums");
  if (reinterpret_cast<uintptr_t>(sums) & 7u)
    return set_error(AWQ_E_INVALID, "act_stats_accumulate: sums must be 8-byte aligned");
  // check_stats wants a non-null abar; the sums stand in for it
  awq_status s = check_stats(X, x_dtype, T, K, reinterpret_cast<const float*>(sums), ws, ws_bytes);
  if (s != AWQ_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t chunks = stats_chunks(T, K, x_dtype);
  AWQ_HIP(timed(AWQ_K_STATS, st,
                [&] {
                  return launch_stats_accumulate(X, dt(x_dtype), T, K, chunks,
                                                 static_cast<double*>(ws), sums, st);
                }),
          "act_stats_accumulate");
  return AWQ_OK;
}

extern "C" awq_status awq_act_stats_finalize(const double* sums, int64_t count, int64_t K,
                                             float* abar, void* stream) {
  awq_status s = check_stats_finalize(sums, count, K, abar);
  if (s != AWQ_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  AWQ_HIP(launch_stats_divide(sums, count, K, abar, st), "act_stats_finalize");
  return AWQ_OK;
}

extern "C" awq_status awq_scale_table(const float* abar, int64_t K, const float* alphas,
                                      int32_t n_alpha, float* s_table, void* stream) {
  awq_status s = check_scale_table(abar, K, alphas, n_alpha, s_table);
  if (s != AWQ_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  AWQ_HIP(timed(AWQ_K_SCALE, st,
                [&] { return launch_scale_table(abar, K, alphas, n_alpha, s_table, nullptr, st); }),
          "scale_table");
  return AWQ_OK;
}

extern "C" awq_status awq_gram_build(const void* X, awq_dtype dtype, int64_t T, int64_t K,
                                     void* G, size_t G_bytes, void* ws, size_t ws_bytes,
                                     void* stream) {
  awq_status s = check_gram_build(X, dtype, T, K, G, G_bytes, ws, ws_bytes);
  if (s != AWQ_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const GramBuildLayout B = gram_build_layout(T, K);
  float* P = at<float>(ws, B.gp);
  AWQ_HIP(timed(AWQ_K_GRAM_BUILD, st,
                [&] {
                  return launch_gram_build(X, T, K, B.Tp, B.S, P, B.ldg, static_cast<uint16_t*>(G),
                                           st);
                }),
          "gram_build");
  return AWQ_OK;
}

namespace {

// Builds G = XᵀX (upper tiles, hi/lo) into the workspace of a Gram search.
awq_status build_gram(const void* X, int64_t T, int64_t K, const SearchLayout& L, void* ws,
                      hipStream_t st) {
  float* P = at<float>(ws, L.gp);
  uint16_t* Gs = at<uint16_t>(ws, L.gs);
  AWQ_HIP(timed(AWQ_K_GRAM_BUILD, st,
                [&] { return launch_gram_build(X, T, K, L.Tp, L.S, P, L.ldg, Gs, st); }),
          "gram_build");
  return AWQ_OK;
}

// α search over the layers of `seg` (one layer, or several reading the same
// X), already validated; N is their total output channels. op selects the
// direct or the Gram candidate GEMM.
awq_status search_scale_impl(int op, const void* X, const Segment* seg, int n_seg,
                             awq_dtype dtype, int64_t T, int64_t N, int64_t K, const float* abar,
                             const float* alphas, int32_t n_alpha, awq_qconfig qc, float* s_best,
                             float* alpha_best, double* mse, double* row_sums, void* ws,
                             int32_t nb, hipStream_t st) {
  const SearchLayout L = search_layout(layout_op(op, qc, dtype), T, N, K, n_alpha, nb, dtype);
  const uint16_t* Gs = nullptr;
  if (builds_gram(op)) {
    awq_status g = build_gram(X, T, K, L, ws, st);
    if (g != AWQ_OK) return g;
    Gs = at<uint16_t>(ws, L.gs);
  } else if (is_gram_op(op)) {
    Gs = static_cast<const uint16_t*>(X);   // a prepared G passed in place of X
  }
  float* s_table = at<float>(ws, L.s_table);
  float* inv_table = at<float>(ws, L.inv);
  double* rs = at<double>(ws, L.row_sums);
  double* mse_dev = at<double>(ws, L.mse);

  AWQ_HIP(timed(AWQ_K_SCALE, st,
                [&] {
                  return launch_scale_table(abar, K, alphas, n_alpha, s_table, inv_table, st);
                }),
          "scale_table");
  for (int c0 = 0; c0 < n_alpha; c0 += nb) {
    const int cb = n_alpha - c0 < nb ? n_alpha - c0 : nb;
    awq_status s = run_batch(X, seg, n_seg, dtype, T, N, K, s_table + int64_t(c0) * K,
                             inv_table + int64_t(c0) * K, K, nullptr, cb, qc, L, ws,
                             rs + int64_t(c0) * N, st, Gs);
    if (s != AWQ_OK) return s;
  }
  AWQ_HIP(timed(AWQ_K_REDUCE, st,
                [&] { return launch_curve(rs, n_alpha, N, double(T) * double(N), mse_dev, st); }),
          "curve");
  AWQ_HIP(hipMemcpyAsync(mse, mse_dev, sizeof(double) * size_t(n_alpha), hipMemcpyDeviceToHost, st),
          "copy mse");
  AWQ_HIP(hipStreamSynchronize(st), "synchronize");
  // a NaN or Inf in X, W or abar (or a sum beyond the float range) makes the
  // curve non-finite and the argmin meaningless: report it, curve written
  for (int i = 0; i < n_alpha; ++i)
    if (!std::isfinite(mse[i]))
      return set_error(AWQ_E_RANGE,
                       "search_scale: output error of alpha #%d is not finite (NaN or Inf in "
                       "the inputs?)", i);
  int best = 0;
  for (int i = 1; i < n_alpha; ++i)
    if (mse[i] < mse[best]) best = i;
  *alpha_best = alphas[best];
  AWQ_HIP(hipMemcpyAsync(s_best, s_table + int64_t(best) * K, sizeof(float) * size_t(K),
                         hipMemcpyDeviceToDevice, st),
          "copy s_best");
  if (row_sums)
    AWQ_HIP(hipMemcpyAsync(row_sums, rs, sizeof(double) * size_t(n_alpha) * size_t(N),
                           hipMemcpyDeviceToDevice, st),
            "copy row_sums");
  AWQ_HIP(hipStreamSynchronize(st), "synchronize");
  return AWQ_OK;
}

}  // namespace

extern "C" awq_status awq_search_scale(const void* X, const void* W, awq_dtype dtype, int64_t T,
                                       int64_t N, int64_t K, const float* abar,
                                       const float* alphas, int32_t n_alpha, awq_qconfig qc,
                                       float* s_best, float* alpha_best, double* mse,
                                       double* row_sums, void* ws, size_t ws_bytes,
                                       void* stream) {
  int32_t nb = 0;
  awq_status s = check_search(AWQ_OP_SEARCH_SCALE, X, W, dtype, T, N, K, abar, alphas, n_alpha,
                              qc, s_best, alpha_best, mse, ws, ws_bytes, &nb);
  if (s != AWQ_OK) return s;
  const Segment seg{W, N, 0};
  return search_scale_impl(AWQ_OP_SEARCH_SCALE, X, &seg, 1, dtype, T, N, K, abar, alphas,
                           n_alpha, qc, s_best, alpha_best, mse, row_sums, ws, nb,
                           static_cast<hipStream_t>(stream));
}

extern "C" awq_status awq_search_scale_gram(const void* X, const void* W, awq_dtype dtype,
                                            int64_t T, int64_t N, int64_t K, const float* abar,
                                            const float* alphas, int32_t n_alpha,
                                            awq_qconfig qc, float* s_best, float* alpha_best,
                                            double* mse, double* row_sums, void* ws,
                                            size_t ws_bytes, void* stream) {
  int32_t nb = 0;
  awq_status s = check_search(AWQ_OP_SEARCH_SCALE_GRAM, X, W, dtype, T, N, K, abar, alphas,
                              n_alpha, qc, s_best, alpha_best, mse, ws, ws_bytes, &nb);
  if (s != AWQ_OK) return s;
  const Segment seg{W, N, 0};
  return search_scale_impl(AWQ_OP_SEARCH_SCALE_GRAM, X, &seg, 1, dtype, T, N, K, abar, alphas,
                           n_alpha, qc, s_best, alpha_best, mse, row_sums, ws, nb,
                           static_cast<hipStream_t>(stream));
}

namespace {

awq_status search_scale_group_op(int op, const void* X, const void* const* W, const int64_t* N,
                                 int32_t n_layers, awq_dtype dtype, int64_t T, int64_t K,
                                 const float* abar, const float* alphas, int32_t n_alpha,
                                 awq_qconfig qc, float* s_best, float* alpha_best, double* mse,
                                 double* row_sums, void* ws, size_t ws_bytes, void* stream) {
  int64_t N_total = 0;
  awq_status s = check_group(W, N, n_layers, &N_total);
  if (s != AWQ_OK) return s;
  if (qc.flags & AWQ_SEARCH_FUSED)
    return set_error(AWQ_E_UNSUPPORTED,
                     "search_scale_group: the fused search covers single-layer searches");
  int32_t nb = 0;
  s = check_search(op, X, W[0], dtype, T, N_total, K, abar, alphas, n_alpha, qc, s_best,
                   alpha_best, mse, ws, ws_bytes, &nb);
  if (s != AWQ_OK) return s;
  Segment seg[kMaxLayers];
  int64_t row0 = 0;
  for (int l = 0; l < n_layers; ++l) {
    seg[l] = Segment{W[l], N[l], row0};
    row0 += N[l];
  }
  return search_scale_impl(op, X, seg, n_layers, dtype, T, N_total, K, abar, alphas, n_alpha,
                           qc, s_best, alpha_best, mse, row_sums, ws, nb,
                           static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" awq_status awq_search_scale_group(const void* X, const void* const* W,
                                             const int64_t* N, int32_t n_layers, awq_dtype dtype,
                                             int64_t T, int64_t K, const float* abar,
                                             const float* alphas, int32_t n_alpha,
                                             awq_qconfig qc, float* s_best, float* alpha_best,
                                             double* mse, double* row_sums, void* ws,
                                             size_t ws_bytes, void* stream) {
  return search_scale_group_op(AWQ_OP_SEARCH_SCALE, X, W, N, n_layers, dtype, T, K, abar, alphas,
                               n_alpha, qc, s_best, alpha_best, mse, row_sums, ws, ws_bytes,
                               stream);
}

extern "C" awq_status awq_search_scale_group_gram(const void* X, const void* const* W,
                                                  const int64_t* N, int32_t n_layers,
                                                  awq_dtype dtype, int64_t T, int64_t K,
                                                  const float* abar, const float* alphas,
                                                  int32_t n_alpha, awq_qconfig qc, float* s_best,
                                                  float* alpha_best, double* mse,
                                                  double* row_sums, void* ws, size_t ws_bytes,
                                                  void* stream) {
  return search_scale_group_op(AWQ_OP_SEARCH_SCALE_GRAM, X, W, N, n_layers, dtype, T, K, abar,
                               alphas, n_alpha, qc, s_best, alpha_best, mse, row_sums, ws,
                               ws_bytes, stream);
}

extern "C" awq_status awq_search_scale_gram_g(const void* G, const void* W, awq_dtype dtype,
                                              int64_t T, int64_t N, int64_t K, const float* abar,
                                              const float* alphas, int32_t n_alpha,
                                              awq_qconfig qc, float* s_best, float* alpha_best,
                                              double* mse, double* row_sums, void* ws,
                                              size_t ws_bytes, void* stream) {
  int32_t nb = 0;
  awq_status s = check_search(AWQ_OP_SEARCH_SCALE_GRAM_G, G, W, dtype, T, N, K, abar, alphas,
                              n_alpha, qc, s_best, alpha_best, mse, ws, ws_bytes, &nb);
  if (s != AWQ_OK) return s;
  const Segment seg{W, N, 0};
  return search_scale_impl(AWQ_OP_SEARCH_SCALE_GRAM_G, G, &seg, 1, dtype, T, N, K, abar, alphas,
                           n_alpha, qc, s_best, alpha_best, mse, row_sums, ws, nb,
                           static_cast<hipStream_t>(stream));
}

extern "C" awq_status awq_search_scale_group_gram_g(const void* G, const void* const* W,
                                                    const int64_t* N, int32_t n_layers,
                                                    awq_dtype dtype, int64_t T, int64_t K,
                                                    const float* abar, const float* alphas,
                                                    int32_t n_alpha, awq_qconfig qc,
                                                    float* s_best, float* alpha_best, double* mse,
                                                    double* row_sums, void* ws, size_t ws_bytes,
                                                    void* stream) {
  return search_scale_group_op(AWQ_OP_SEARCH_SCALE_GRAM_G, G, W, N, n_layers, dtype, T, K, abar,
                               alphas, n_alpha, qc, s_best, alpha_best, mse, row_sums, ws,
                               ws_bytes, stream);
}

namespace {

awq_status search_clip_impl(int op, const void* X, const void* W, awq_dtype dtype, int64_t T,
                            int64_t N, int64_t K, const float* s, const float* ratios,
                            int32_t n_ratio, awq_qconfig qc, float* ratio_best, double* mse_clip,
                            double* row_sums, void* ws, int32_t nb, hipStream_t st) {
  const SearchLayout L = search_layout(layout_op(op, qc, dtype), T, N, K, n_ratio, nb, dtype);
  double* rs = at<double>(ws, L.row_sums);
  double* best = at<double>(ws, L.best);
  double* mc = at<double>(ws, L.scalar);
  float* inv = at<float>(ws, L.inv);
  float* s_copy = at<float>(ws, L.s_table);
  const Segment seg{W, N, 0};
  const uint16_t* Gs = nullptr;
  if (builds_gram(op)) {
    awq_status g = build_gram(X, T, K, L, ws, st);
    if (g != AWQ_OK) return g;
    Gs = at<uint16_t>(ws, L.gs);
  } else if (is_gram_op(op)) {
    Gs = static_cast<const uint16_t*>(X);   // a prepared G passed in place of X
  }
  AWQ_HIP(timed(AWQ_K_SCALE, st, [&] { return launch_reciprocal(s, K, s_copy, inv, st); }),
          "reciprocal");
  for (int c0 = 0; c0 < n_ratio; c0 += nb) {
    const int cb = n_ratio - c0 < nb ? n_ratio - c0 : nb;
    awq_status st_ = run_batch(X, &seg, 1, dtype, T, N, K, s_copy, inv, 0, ratios + c0, cb, qc,
                               L, ws, rs + int64_t(c0) * N, st, Gs);
    if (st_ != AWQ_OK) return st_;
  }
  AWQ_HIP(timed(AWQ_K_REDUCE, st,
                [&] {
                  return launch_clip_select(rs, n_ratio, N, ratios, double(T) * double(N),
                                            ratio_best, best, mc, st);
                }),
          "clip_select");
  if (row_sums)
    AWQ_HIP(hipMemcpyAsync(row_sums, rs, sizeof(double) * size_t(n_ratio) * size_t(N),
                           hipMemcpyDeviceToDevice, st),
            "copy row_sums");
  AWQ_HIP(hipMemcpyAsync(mse_clip, mc, sizeof(double), hipMemcpyDeviceToHost, st), "copy mse_clip");
  AWQ_HIP(hipStreamSynchronize(st), "synchronize");
  if (!std::isfinite(*mse_clip))
    return set_error(AWQ_E_RANGE,
                     "search_clip: output error is not finite (NaN or Inf in the inputs?)");
  return AWQ_OK;
}

}  // namespace

extern "C" awq_status awq_search_clip(const void* X, const void* W, awq_dtype dtype, int64_t T,
                                      int64_t N, int64_t K, const float* s, const float* ratios,
                                      int32_t n_ratio, awq_qconfig qc, float* ratio_best,
                                      double* mse_clip, double* row_sums, void* ws,
                                      size_t ws_bytes, void* stream) {
  int32_t nb = 0;
  awq_status st_ = check_search(AWQ_OP_SEARCH_CLIP, X, W, dtype, T, N, K, s, ratios, n_ratio, qc,
                                ratio_best, mse_clip, nullptr, ws, ws_bytes, &nb);
  if (st_ != AWQ_OK) return st_;
  return search_clip_impl(AWQ_OP_SEARCH_CLIP, X, W, dtype, T, N, K, s, ratios, n_ratio, qc,
                          ratio_best, mse_clip, row_sums, ws, nb,
                          static_cast<hipStream_t>(stream));
}

extern "C" awq_status awq_search_clip_gram(const void* X, const void* W, awq_dtype dtype,
                                           int64_t T, int64_t N, int64_t K, const float* s,
                                           const float* ratios, int32_t n_ratio, awq_qconfig qc,
                                           float* ratio_best, double* mse_clip, double* row_sums,
                                           void* ws, size_t ws_bytes, void* stream) {
  int32_t nb = 0;
  awq_status st_ = check_search(AWQ_OP_SEARCH_CLIP_GRAM, X, W, dtype, T, N, K, s, ratios, n_ratio,
                                qc, ratio_best, mse_clip, nullptr, ws, ws_bytes, &nb);
  if (st_ != AWQ_OK) return st_;
  return search_clip_impl(AWQ_OP_SEARCH_CLIP_GRAM, X, W, dtype, T, N, K, s, ratios, n_ratio, qc,
                          ratio_best, mse_clip, row_sums, ws, nb,
                          static_cast<hipStream_t>(stream));
}

extern "C" awq_status awq_search_clip_gram_g(const void* G, const void* W, awq_dtype dtype,
                                             int64_t T, int64_t N, int64_t K, const float* s,
                                             const float* ratios, int32_t n_ratio,
                                             awq_qconfig qc, float* ratio_best, double* mse_clip,
                                             double* row_sums, void* ws, size_t ws_bytes,
                                             void* stream) {
  int32_t nb = 0;
  awq_status st_ = check_search(AWQ_OP_SEARCH_CLIP_GRAM_G, G, W, dtype, T, N, K, s, ratios,
                                n_ratio, qc, ratio_best, mse_clip, nullptr, ws, ws_bytes, &nb);
  if (st_ != AWQ_OK) return st_;
  return search_clip_impl(AWQ_OP_SEARCH_CLIP_GRAM_G, G, W, dtype, T, N, K, s, ratios, n_ratio,
                          qc, ratio_best, mse_clip, row_sums, ws, nb,
                          static_cast<hipStream_t>(stream));
}

extern "C" awq_status awq_quantize_pack(const void* W, awq_dtype w_dtype, int64_t N, int64_t K,
                                        const float* s, const float* ratio, awq_qconfig qc,
                                        int32_t* qweight, int32_t* qzeros, uint16_t* scales,
                                        void* ws, size_t ws_bytes, void* stream) {
  awq_status s_ = check_pack(W, w_dtype, N, K, s, qc, qweight, qzeros, scales, ws, ws_bytes);
  if (s_ != AWQ_OK) return s_;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int* flag = static_cast<int*>(ws);
  AWQ_HIP(hipMemsetAsync(flag, 0, sizeof(int), st), "clear overflow flag");
  AWQ_HIP(timed(AWQ_K_PACK, st,
                [&] {
                  return launch_pack(W, dt(w_dtype), N, K, s, ratio, qc.w_bit, qc.group_size,
                                     qc.zero_point, qweight, qzeros, scales, flag, st);
                }),
          "pack");
  int host_flag = 0;
  AWQ_HIP(hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, st), "copy flag");
  AWQ_HIP(hipStreamSynchronize(st), "synchronize");
  if (host_flag) return set_error(AWQ_E_RANGE, "quantize_pack: a group step overflows fp16");
  return AWQ_OK;
}

extern "C" awq_status awq_fold_norm(void* gamma, void* beta, awq_dtype dtype, int64_t K,
                                    const float* s, void* stream) {
  awq_status st_ = check_fold_norm(gamma, beta, dtype, K, s);
  if (st_ != AWQ_OK) return st_;
  hipStream_t st = static_cast<hipStream_t>(stream);
  AWQ_HIP(timed(AWQ_K_FOLD, st, [&] { return launch_fold_vec(gamma, dt(dtype), K, s, st); }),
          "fold_norm");
  if (beta)
    AWQ_HIP(timed(AWQ_K_FOLD, st, [&] { return launch_fold_vec(beta, dt(dtype), K, s, st); }),
            "fold_norm bias");
  return AWQ_OK;
}

extern "C" awq_status awq_fold_linear(void* W_prev, void* bias_prev, awq_dtype dtype, int64_t K,
                                      int64_t K_prev, const float* s, void* stream) {
  awq_status st_ = check_fold_linear(W_prev, bias_prev, dtype, K, K_prev, s);
  if (st_ != AWQ_OK) return st_;
  hipStream_t st = static_cast<hipStream_t>(stream);
  AWQ_HIP(timed(AWQ_K_FOLD, st,
                [&] { return launch_fold_rows(W_prev, dt(dtype), K, K_prev, s, st); }),
          "fold_linear");
  if (bias_prev)
    AWQ_HIP(timed(AWQ_K_FOLD, st,
                  [&] { return launch_fold_vec(bias_prev, dt(dtype), K, s, st); }),
            "fold_linear bias");
  return AWQ_OK;
}

extern "C" awq_status awq_w4a16_matmul(const void* X, awq_dtype dtype, int64_t T, int64_t N,
                                       int64_t K, const int32_t* qweight, const int32_t* qzeros,
                                       const uint16_t* scales, int32_t group_size, void* Y,
                                       void* ws, size_t ws_bytes, void* stream) {
  awq_status st_ = check_w4a16(X, dtype, T, N, K, qweight, qzeros, scales, group_size, Y, ws,
                               ws_bytes);
  if (st_ != AWQ_OK) return st_;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int f16 = dtype == AWQ_F16;
  const uint16_t* x = static_cast<const uint16_t*>(X);
  uint16_t* y = static_cast<uint16_t*>(Y);
  if (T <= kW4A16GemvMaxT) {
    float* partial = static_cast<float*>(ws);
    const bool mg = w4a16_use_mgemv(N, qweight, qzeros);
    const int64_t kpw = mg ? w4a16_mgemv_kpw(N, K) : w4a16_gemv_kpw(N, K);
    const int64_t chunks = mg ? w4a16_mgemv_chunks(N, K) : w4a16_gemv_chunks(N, K);
    AWQ_HIP(timed(AWQ_K_W4A16, st,
                  [&] {
                    return mg ? launch_w4a16_mgemv(x, T, N, K, qweight, qzeros, scales,
                                                   group_size, f16, kpw, partial, st, 4)
                              : launch_w4a16_gemv(x, T, N, K, qweight, qzeros, scales,
                                                  group_size, f16, kpw, partial, st);
                  }),
            "w4a16 gemv");
    AWQ_HIP(timed(AWQ_K_W4A16_REDUCE, st,
                  [&] { return launch_w4a16_gemv_reduce(partial, chunks, T, N, f16, y, st); }),
            "w4a16 gemv reduce");
    return AWQ_OK;
  }
  if (ws_bytes < awq_w4a16_workspace_bytes(T, N, K, dtype)) {
    // (the checks admitted it only where the fused GEMM fits)
    AWQ_HIP(timed(AWQ_K_W4A16, st,
                  [&] {
                    return launch_w4a16_gemm_q(x, qweight, qzeros, scales, T, N, K, group_size,
                                               f16, y, st);
                  }),
            "w4a16 gemm");
    return AWQ_OK;
  }
  uint16_t* Wd = static_cast<uint16_t*>(ws);
  AWQ_HIP(timed(AWQ_K_DEQUANT, st,
                [&] {
                  return launch_w4a16_dequant(qweight, qzeros, scales, N, K, group_size, f16, Wd,
                                              st);
                }),
          "w4a16 dequant");
  AWQ_HIP(timed(AWQ_K_W4A16, st,
                [&] { return launch_w4a16_gemm(x, Wd, T, N, K, f16, y, st); }),
          "w4a16 gemm");
  return AWQ_OK;
}

extern "C" awq_status awq_w3a16_matmul(const void* X, awq_dtype dtype, int64_t T, int64_t N,
                                       int64_t K, const int32_t* qweight, const int32_t* qzeros,
                                       const uint16_t* scales, int32_t group_size, void* Y,
                                       void* ws, size_t ws_bytes, void* stream) {
  awq_status st_ = check_w3a16(X, dtype, T, N, K, qweight, qzeros, scales, group_size, Y, ws,
                               ws_bytes);
  if (st_ != AWQ_OK) return st_;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int f16 = dtype == AWQ_F16;
  if (T <= kW4A16GemvMaxT) {
    float* partial = static_cast<float*>(ws);
    const int64_t kpw = w4a16_mgemv_kpw(N, K), chunks = w4a16_mgemv_chunks(N, K);
    AWQ_HIP(timed(AWQ_K_W4A16, st,
                  [&] {
                    return launch_w4a16_mgemv(static_cast<const uint16_t*>(X), T, N, K, qweight,
                                              qzeros, scales, group_size, f16, kpw, partial, st,
                                              3);
                  }),
            "w3a16 gemv");
    AWQ_HIP(timed(AWQ_K_W4A16_REDUCE, st,
                  [&] {
                    return launch_w4a16_gemv_reduce(partial, chunks, T, N, f16,
                                                    static_cast<uint16_t*>(Y), st);
                  }),
            "w3a16 gemv reduce");
    return AWQ_OK;
  }
  uint16_t* Wd = static_cast<uint16_t*>(ws);
  AWQ_HIP(timed(AWQ_K_DEQUANT, st,
                [&] {
                  return launch_w3a16_dequant(qweight, qzeros, scales, N, K, group_size, f16, Wd,
                                              st);
                }),
          "w3a16 dequant");
  AWQ_HIP(timed(AWQ_K_W4A16, st,
                [&] {
                  return launch_w4a16_gemm(static_cast<const uint16_t*>(X), Wd, T, N, K, f16,
                                           static_cast<uint16_t*>(Y), st);
                }),
          "w3a16 gemm");
  return AWQ_OK;
}

extern "C" void awq_profile_enable(int on) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  p.on = on != 0;
}

extern "C" void awq_profile_reset(void) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  for (auto& q : p.pending) {
    // the pending timings are discarded; only wait so the events can be reused
    (void)hipEventSynchronize(q.b);
    p.spare.push_back(q.a);
    p.spare.push_back(q.b);
  }
  p.pending.clear();
  for (int i = 0; i < AWQ_K_COUNT; ++i) {
    p.ms[i] = 0.0;
    p.n[i] = 0;
  }
}

extern "C" awq_status awq_profile_read(int kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= AWQ_K_COUNT || !total_ms || !launches)
    return set_error(AWQ_E_INVALID, "profile_read: bad kind or NULL output");
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  for (auto& q : p.pending) {
    hipError_t e = hipEventSynchronize(q.b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, q.a, q.b);
    if (e != hipSuccess) return hip_fail(e, "profile_read");
    p.ms[q.kind] += double(ms);
    p.n[q.kind] += 1;
    p.spare.push_back(q.a);
    p.spare.push_back(q.b);
  }
  p.pending.clear();
  *total_ms = p.ms[kind];
  *launches = p.n[kind];
  return AWQ_OK;
}
