// Step 6 — deterministic float64 reductions of the search GEMM's partials.
//
//   row_sums[c]  = Σ_mt partials[mt][c]            (M_n of candidate c/N, row c%N)
//   mse[a]       = Σ_n row_sums[a·N + n] / (T·N)   ("05 — AWQ", section 4: the
//                                                   output MSE of each candidate)
//   clip select  : per row n, the ratio with the smallest M_n(r) (lowest index
//                  on ties), and Σ_n of those minima / (T·N) ("Optional:
//                  per-channel clipping").
//
// Fixed summation orders and no atomics, so repeated runs are bitwise equal.
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;

// 64 columns per workgroup, 4 lanes per column: lane group g adds token
// tiles g, g+4, ... in order (8 loads in flight), then the four sums are
// added in a fixed order.
__global__ __launch_bounds__(kThreads) void reduce_rows_kernel(const float* __restrict__ partials,
                                                               int64_t MT, int64_t Nc,
                                                               double* __restrict__ row_sums) {
  __shared__ double red[4][64];
  const int cl = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int64_t c = int64_t(blockIdx.x) * 64 + cl;
  double s = 0.0;
  if (c < Nc) {
#pragma unroll 8
    for (int64_t m = g; m < MT; m += 4) s += double(partials[m * Nc + c]);
  }
  red[g][cl] = s;
  __syncthreads();
  if (g == 0 && c < Nc) row_sums[c] = ((red[0][cl] + red[1][cl]) + red[2][cl]) + red[3][cl];
}

// Fixed-shape block sum: thread i adds elements i, i+256, ...; then a tree.
__device__ double block_sum(double v, double* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  return sh[0];
}

__global__ __launch_bounds__(kThreads) void curve_kernel(const double* __restrict__ row_sums,
                                                         int64_t N, double denom,
                                                         double* __restrict__ mse) {
  __shared__ double sh[kThreads];
  const double* r = row_sums + int64_t(blockIdx.x) * N;
  double s = 0.0;
  for (int64_t n = threadIdx.x; n < N; n += kThreads) s += r[n];
  const double tot = block_sum(s, sh);
  if (threadIdx.x == 0) mse[blockIdx.x] = tot / denom;
}

__global__ __launch_bounds__(kThreads) void clip_argmin_kernel(const double* __restrict__ row_sums,
                                                               int n_ratio, int64_t N, GridArgs ratios,
                                                               float* __restrict__ ratio_best,
                                                               double* __restrict__ best) {
  const int64_t n = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (n >= N) return;
  int bi = 0;
  double bv = row_sums[n];
  for (int r = 1; r < n_ratio; ++r) {
    const double v = row_sums[int64_t(r) * N + n];
    if (v < bv) {
      bv = v;
      bi = r;
    }
  }
  ratio_best[n] = ratios.v[bi];
  best[n] = bv;
}

}  // namespace

hipError_t launch_reduce_rows(const float* partials, int64_t MT, int64_t Nc, double* row_sums,
                              hipStream_t st) {
  reduce_rows_kernel<<<unsigned((Nc + 63) / 64), kThreads, 0, st>>>(partials, MT, Nc, row_sums);
  return hipGetLastError();
}

hipError_t launch_curve(const double* row_sums, int n_cand, int64_t N, double denom, double* mse,
                        hipStream_t st) {
  curve_kernel<<<unsigned(n_cand), kThreads, 0, st>>>(row_sums, N, denom, mse);
  return hipGetLastError();
}

hipError_t launch_clip_select(const double* row_sums, int n_ratio, int64_t N,
                              const float* ratios_host, double denom, float* ratio_best,
                              double* best, double* mse_clip, hipStream_t st) {
  GridArgs g{};
  for (int i = 0; i < n_ratio && i < 64; ++i) g.v[i] = ratios_host[i];
  clip_argmin_kernel<<<unsigned((N + kThreads - 1) / kThreads), kThreads, 0, st>>>(
      row_sums, n_ratio, N, g, ratio_best, best);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  curve_kernel<<<1, kThreads, 0, st>>>(best, N, denom, mse_clip);
  return hipGetLastError();
}

}  // namespace awq
