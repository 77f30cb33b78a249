// Step 2 — scale table s[a][j] = ā_j^α_a / sqrt(max_k ā_k^α_a · min_k ā_k^α_a).
//
// "AWQ and Activation-Aware Scaling", section "Scaling instead of protecting":
// s = ā^α with one exponent α in [0, 1] per layer. "05 — AWQ", section 4:
// s_j is the channel's activation magnitude to the power α times a constant;
// the constant here is one per α, the reciprocal geometric mean of the
// largest and smallest scale. Since x^α is increasing for α >= 0, the largest
// and smallest ā^α are the powers of the largest and smallest ā. float64
// throughout, one rounding to float32. Tiny: one workgroup.
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 1024;
constexpr double kAbarFloor = 1e-8;

__global__ __launch_bounds__(kThreads) void scale_table_kernel(const float* __restrict__ abar,
                                                               int64_t K, GridArgs alphas, int n,
                                                               float* __restrict__ s_table) {
  __shared__ double smax[kThreads], smin[kThreads];
  double lo = 1e300, hi = 0.0;
  for (int64_t j = threadIdx.x; j < K; j += kThreads) {
    const double a = fmax(double(abar[j]), kAbarFloor);
    lo = fmin(lo, a);
    hi = fmax(hi, a);
  }
  smax[threadIdx.x] = hi;
  smin[threadIdx.x] = lo;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      smax[threadIdx.x] = fmax(smax[threadIdx.x], smax[threadIdx.x + w]);
      smin[threadIdx.x] = fmin(smin[threadIdx.x], smin[threadIdx.x + w]);
    }
    __syncthreads();
  }
  const double amax = smax[0], amin = smin[0];
  for (int i = 0; i < n; ++i) {
    const double al = double(alphas.v[i]);
    const double norm = sqrt(pow(amax, al) * pow(amin, al));
    for (int64_t j = threadIdx.x; j < K; j += kThreads) {
      const double a = fmax(double(abar[j]), kAbarFloor);
      s_table[int64_t(i) * K + j] = float(pow(a, al) / norm);
    }
  }
}

}  // namespace

hipError_t launch_scale_table(const float* abar, int64_t K, const float* alphas_host, int n,
                              float* s_table, hipStream_t st) {
  GridArgs g{};
  for (int i = 0; i < n && i < 64; ++i) g.v[i] = alphas_host[i];
  scale_table_kernel<<<1, kThreads, 0, st>>>(abar, K, g, n, s_table);
  return hipGetLastError();
}

}  // namespace awq
