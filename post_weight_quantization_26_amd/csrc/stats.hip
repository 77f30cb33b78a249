// Step 1 — per-input-channel mean activation magnitude ā_j = Σ_t |x_tj| / T.
//
// "AWQ and Activation-Aware Scaling", section "Scaling instead of protecting":
// the scale follows the per-channel mean activation magnitude. "05 — AWQ",
// section 4: the statistic is gathered from a small calibration set.
//
// HBM-bound column reduction. A workgroup owns a strip of 64·VEC columns (VEC
// = 16 bytes of elements per lane, so a wavefront reads whole 1 KiB row
// segments) and one chunk of tokens; its 4 wavefronts take interleaved rows of
// the chunk, 4 row loads in flight per lane. Sums are float64 (exact for bf16
// and f16 inputs, so the result does not depend on the split). The 4 row
// lanes meet in LDS; one float64 partial per (chunk, column) goes to the
// workspace, and a finalise pass adds the chunks in a fixed order and rounds
// once to float32.
#include <mutex>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

// The float64 chunk partials of awq_act_stats_noalloc, for callers that
// cannot allocate: one copy per device, held until the process ends, shared
// by every such call on that device. Every entry a launch reads is written
// by the same launch first, so nothing needs clearing.
static __device__ __align__(256) double scratch[kStatsScratchDoubles];

namespace {

constexpr int kColThreads = 64;
constexpr int kRowLanes = 4;
constexpr int kUnroll = 4;

template <int DT>
struct Elem;
template <>
struct Elem<0> {  // f32
  static constexpr int VEC = 4;
  __device__ static void abs_add(const uint4& q, double (&acc)[VEC]) {
    acc[0] += fabs(double(__uint_as_float(q.x)));
    acc[1] += fabs(double(__uint_as_float(q.y)));
    acc[2] += fabs(double(__uint_as_float(q.z)));
    acc[3] += fabs(double(__uint_as_float(q.w)));
  }
};
template <>
struct Elem<1> {  // bf16
  static constexpr int VEC = 8;
  __device__ static void abs_add(const uint4& q, double (&acc)[VEC]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += fabs(double(__uint_as_float(w[i] << 16)));
      acc[2 * i + 1] += fabs(double(__uint_as_float(w[i] & 0xFFFF0000u)));
    }
  }
};
template <>
struct Elem<2> {  // f16
  static constexpr int VEC = 8;
  __device__ static void abs_add(const uint4& q, double (&acc)[VEC]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += fabs(double(f16_to_f32(uint16_t(w[i] & 0xFFFFu))));
      acc[2 * i + 1] += fabs(double(f16_to_f32(uint16_t(w[i] >> 16))));
    }
  }
};

// X is read exactly once here: non-temporal 16-byte loads stream it past the
// caches (measured on MI355X: ~7.0 TB/s against ~6.3 TB/s for ordinary loads).
__device__ __forceinline__ uint4 load_stream(const char* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

template <int DT>
__global__ __launch_bounds__(kColThreads* kRowLanes) void stats_partial_kernel(
    const uint16_t* __restrict__ X16, int64_t T, int64_t K, int64_t rows_per_chunk,
    double* __restrict__ partial) {
  constexpr int VEC = Elem<DT>::VEC;
  constexpr int ESZ = 16 / VEC;
  __shared__ double red[kRowLanes - 1][kColThreads * VEC];

  const int tc = threadIdx.x % kColThreads;
  const int rl = threadIdx.x / kColThreads;
  const int64_t col0 = (int64_t(blockIdx.x) * kColThreads + tc) * VEC;
  const int64_t chunk = blockIdx.y;
  const int64_t r_begin = chunk * rows_per_chunk;
  const int64_t r_end = min(T, r_begin + rows_per_chunk);
  const bool active = col0 < K;
  const char* base = reinterpret_cast<const char*>(X16);

  double acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.0;

  if (active) {
    int64_t r = r_begin + rl;
    // Main loop: kUnroll independent 16-byte loads per lane in flight.
    for (; r + (kUnroll - 1) * kRowLanes < r_end; r += kUnroll * kRowLanes) {
      uint4 q[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        q[u] = load_stream(base + ((r + u * kRowLanes) * K + col0) * ESZ);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) Elem<DT>::abs_add(q[u], acc);
    }
    for (; r < r_end; r += kRowLanes) {
      const uint4 q = load_stream(base + (r * K + col0) * ESZ);
      Elem<DT>::abs_add(q, acc);
    }
  }
  if (rl > 0) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) red[rl - 1][tc * VEC + i] = acc[i];
  }
  __syncthreads();
  if (rl == 0 && active) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      double s = acc[i];
#pragma unroll
      for (int l = 0; l < kRowLanes - 1; ++l) s += red[l][tc * VEC + i];
      partial[chunk * K + col0 + i] = s;
    }
  }
}

// Finalise: 64 columns per workgroup, 4 lanes per column each adding every
// 4th chunk in order, then the 4 sums in a fixed order; one rounding to f32.
__global__ __launch_bounds__(256) void stats_finalize_kernel(const double* __restrict__ partial,
                                                             int64_t chunks, int64_t T, int64_t K,
                                                             float* __restrict__ abar) {
  __shared__ double red[4][64];
  const int cl = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int64_t j = int64_t(blockIdx.x) * 64 + cl;
  double s = 0.0;
  if (j < K) {
#pragma unroll 4
    for (int64_t c = g; c < chunks; c += 4) s += partial[c * K + j];
  }
  red[g][cl] = s;
  __syncthreads();
  if (g == 0 && j < K) abar[j] = float((((red[0][cl] + red[1][cl]) + red[2][cl]) + red[3][cl]) / double(T));
}

// Calibration in batches: sums[j] += this batch's column sum, formed from the
// chunk partials exactly as stats_finalize_kernel forms it.
__global__ __launch_bounds__(256) void stats_accumulate_kernel(const double* __restrict__ partial,
                                                               int64_t chunks, int64_t K,
                                                               double* __restrict__ sums) {
  __shared__ double red[4][64];
  const int cl = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int64_t j = int64_t(blockIdx.x) * 64 + cl;
  double s = 0.0;
  if (j < K) {
#pragma unroll 4
    for (int64_t c = g; c < chunks; c += 4) s += partial[c * K + j];
  }
  red[g][cl] = s;
  __syncthreads();
  if (g == 0 && j < K) sums[j] += ((red[0][cl] + red[1][cl]) + red[2][cl]) + red[3][cl];
}

__global__ __launch_bounds__(256) void stats_divide_kernel(const double* __restrict__ sums,
                                                           int64_t count, int64_t K,
                                                           float* __restrict__ abar) {
  const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (j < K) abar[j] = float(sums[j] / double(count));
}

}  // namespace

hipError_t launch_stats_accumulate(const void* X, int dtype, int64_t T, int64_t K,
                                   int64_t chunks, double* partial, double* sums,
                                   hipStream_t st) {
  const int vec = dtype == 0 ? 4 : 8;
  const int64_t rows_per_chunk = (T + chunks - 1) / chunks;
  dim3 grid(unsigned((K + int64_t(kColThreads) * vec - 1) / (int64_t(kColThreads) * vec)),
            unsigned(chunks));
  dim3 block(kColThreads * kRowLanes);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (dtype == 0)
    stats_partial_kernel<0><<<grid, block, 0, st>>>(x, T, K, rows_per_chunk, partial);
  else if (dtype == 1)
    stats_partial_kernel<1><<<grid, block, 0, st>>>(x, T, K, rows_per_chunk, partial);
  else
    stats_partial_kernel<2><<<grid, block, 0, st>>>(x, T, K, rows_per_chunk, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  stats_accumulate_kernel<<<unsigned((K + 63) / 64), 256, 0, st>>>(partial, chunks, K, sums);
  return hipGetLastError();
}

hipError_t launch_stats_divide(const double* sums, int64_t count, int64_t K, float* abar,
                               hipStream_t st) {
  stats_divide_kernel<<<unsigned((K + 255) / 256), 256, 0, st>>>(sums, count, K, abar);
  return hipGetLastError();
}

// Device address of `scratch` on the current device. In host code the
// array's name is only a stand-in, so its address is looked up once per
// device (with that device current) and kept.
hipError_t stats_scratch(double** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptr[dev] = p;
  }
  *out = static_cast<double*>(ptr[dev]);
  return hipSuccess;
}

hipError_t launch_stats(const void* X, int dtype, int64_t T, int64_t K, int64_t chunks,
                        double* partial, float* abar, hipStream_t st) {
  const int vec = dtype == 0 ? 4 : 8;
  const int64_t rows_per_chunk = (T + chunks - 1) / chunks;
  dim3 grid(unsigned((K + int64_t(kColThreads) * vec - 1) / (int64_t(kColThreads) * vec)),
            unsigned(chunks));
  dim3 block(kColThreads * kRowLanes);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (dtype == 0)
    stats_partial_kernel<0><<<grid, block, 0, st>>>(x, T, K, rows_per_chunk, partial);
  else if (dtype == 1)
    stats_partial_kernel<1><<<grid, block, 0, st>>>(x, T, K, rows_per_chunk, partial);
  else
    stats_partial_kernel<2><<<grid, block, 0, st>>>(x, T, K, rows_per_chunk, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  stats_finalize_kernel<<<unsigned((K + 63) / 64), 256, 0, st>>>(partial, chunks, T, K, abar);
  return hipGetLastError();
}

}  // namespace awq
