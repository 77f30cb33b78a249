// Step 2 — scale table s[a][j] = ā_j^α_a / sqrt(max_k ā_k^α_a · min_k ā_k^α_a).
//
// "AWQ and Activation-Aware Scaling", section "Scaling instead of protecting":
// s = ā^α with one exponent α in [0, 1] per layer. "05 — AWQ: Activation-Aware
// Weight Scaling", section 4: s_j is the channel's activation magnitude to the
// power α times a constant; the constant here is one per α, the reciprocal
// geometric mean of the largest and smallest scale. Since x^α is increasing
// for α >= 0, the largest and smallest ā^α are the powers of the largest and
// smallest ā. float64 throughout, one rounding to float32.
//
// Grid: (column blocks, α). Every workgroup finds max/min ā itself (K values,
// L2-resident) so no second launch is needed. The reciprocal table 1/s used
// by the candidate transform is written alongside; for the clip search a
// companion kernel copies the fixed scale row and its reciprocals.
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr double kAbarFloor = 1e-8;

__global__ __launch_bounds__(kThreads) void scale_table_kernel(const float* __restrict__ abar,
                                                               int64_t K, GridArgs alphas,
                                                               float* __restrict__ s_table,
                                                               float* __restrict__ inv_table) {
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
  const int i = blockIdx.y;
  const double al = double(alphas.v[i]);
  const double norm = sqrt(pow(smax[0], al) * pow(smin[0], al));
  const int64_t j = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (j < K) {
    const double a = fmax(double(abar[j]), kAbarFloor);
    const float s = float(pow(a, al) / norm);
    s_table[int64_t(i) * K + j] = s;
    if (inv_table) inv_table[int64_t(i) * K + j] = 1.0f / s;
  }
}

// Aligned copy of a scale row and its reciprocals.
__global__ __launch_bounds__(kThreads) void reciprocal_kernel(const float* __restrict__ s,
                                                              int64_t n, float* __restrict__ s_copy,
                                                              float* __restrict__ inv) {
  const int64_t j = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (j < n) {
    const float v = s[j];
    s_copy[j] = v;
    inv[j] = 1.0f / v;
  }
}

}  // namespace

hipError_t launch_scale_table(const float* abar, int64_t K, const float* alphas_host, int n,
                              float* s_table, float* inv_table, hipStream_t st) {
  GridArgs g{};
  for (int i = 0; i < n && i < 64; ++i) g.v[i] = alphas_host[i];
  dim3 grid(unsigned((K + kThreads - 1) / kThreads), unsigned(n));
  scale_table_kernel<<<grid, kThreads, 0, st>>>(abar, K, g, s_table, inv_table);
  return hipGetLastError();
}

hipError_t launch_reciprocal(const float* s, int64_t n, float* s_copy, float* inv,
                             hipStream_t st) {
  reciprocal_kernel<<<unsigned((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(s, n, s_copy,
                                                                                 inv);
  return hipGetLastError();
}

}  // namespace awq
