// The fold: divide the operation that produces a layer's input by the chosen
// per-input-channel scale s, in place, so that the scaled weights W·diag(s)
// see X·diag(s)^-1 with no extra operation at run time ("AWQ and
// Activation-Aware Scaling", sections "Scaling instead of protecting" and
// "When it breaks": the division goes into the preceding normalisation's
// per-channel weights, or into a preceding linear layer).
//
//   norm:   γ_j ← γ_j / s_j,  β_j ← β_j / s_j              (vectors of K)
//   linear: W_prev[j][:] ← W_prev[j][:] / s_j, b_j ← b_j / s_j  (W_prev [K, K_prev])
//
// Each element is one IEEE float32 division of its float32 value, converted
// once to the storage type with round-to-nearest-even (hardware conversions).
// HBM-bound elementwise work: the row kernel moves 16 bytes per lane.
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;

template <int DT>
__device__ __forceinline__ float load1(const void* p, int64_t i) {
  if constexpr (DT == 0) return static_cast<const float*>(p)[i];
  else if constexpr (DT == 1) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return f16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <int DT>
__device__ __forceinline__ uint32_t to_bits(float f) {
  if constexpr (DT == 1) return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
  else return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

template <int DT>
__device__ __forceinline__ void store1(void* p, int64_t i, float f) {
  if constexpr (DT == 0) static_cast<float*>(p)[i] = f;
  else static_cast<uint16_t*>(p)[i] = uint16_t(to_bits<DT>(f));
}

// v[j] ← v[j] / s[j] for j < K (norm weight, norm bias, previous linear's bias).
template <int DT>
__global__ __launch_bounds__(kThreads) void fold_vec_kernel(void* __restrict__ v, int64_t K,
                                                            const float* __restrict__ s) {
  const int64_t j = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (j < K) store1<DT>(v, j, load1<DT>(v, j) / s[j]);
}

// Row j of W [K, K_prev] divided by s[j]. A lane owns 16 bytes of one row
// (K_prev·elem_size is a multiple of 16, so a lane never straddles rows).
template <int DT>
__global__ __launch_bounds__(kThreads) void fold_rows_kernel(void* __restrict__ W, int64_t K,
                                                             int64_t K_prev,
                                                             const float* __restrict__ s) {
  constexpr int VEC = DT == 0 ? 4 : 8;
  const int64_t e0 = (int64_t(blockIdx.x) * kThreads + threadIdx.x) * VEC;
  if (e0 >= K * K_prev) return;
  const float d = s[e0 / K_prev];
  uint4* p = reinterpret_cast<uint4*>(static_cast<char*>(W) + e0 * (DT == 0 ? 4 : 2));
  uint4 q = *p;
  if constexpr (DT == 0) {
    q.x = __float_as_uint(__uint_as_float(q.x) / d);
    q.y = __float_as_uint(__uint_as_float(q.y) / d);
    q.z = __float_as_uint(__uint_as_float(q.z) / d);
    q.w = __float_as_uint(__uint_as_float(q.w) / d);
  } else {
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = DT == 1 ? bf16_to_f32(uint16_t(w[i] & 0xFFFFu)) : f16_to_f32(uint16_t(w[i] & 0xFFFFu));
      const float hi = DT == 1 ? bf16_to_f32(uint16_t(w[i] >> 16)) : f16_to_f32(uint16_t(w[i] >> 16));
      w[i] = to_bits<DT>(lo / d) | (to_bits<DT>(hi / d) << 16);
    }
    q.x = w[0]; q.y = w[1]; q.z = w[2]; q.w = w[3];
  }
  *p = q;
}

}  // namespace

hipError_t launch_fold_vec(void* v, int dtype, int64_t K, const float* s, hipStream_t st) {
  const unsigned blocks = unsigned((K + kThreads - 1) / kThreads);
  if (dtype == 0)
    fold_vec_kernel<0><<<blocks, kThreads, 0, st>>>(v, K, s);
  else if (dtype == 1)
    fold_vec_kernel<1><<<blocks, kThreads, 0, st>>>(v, K, s);
  else
    fold_vec_kernel<2><<<blocks, kThreads, 0, st>>>(v, K, s);
  return hipGetLastError();
}

hipError_t launch_fold_rows(void* W, int dtype, int64_t K, int64_t K_prev, const float* s,
                            hipStream_t st) {
  const int64_t vec = dtype == 0 ? 4 : 8;
  const int64_t lanes = K * K_prev / vec;
  const unsigned blocks = unsigned((lanes + kThreads - 1) / kThreads);
  if (dtype == 0)
    fold_rows_kernel<0><<<blocks, kThreads, 0, st>>>(W, K, K_prev, s);
  else if (dtype == 1)
    fold_rows_kernel<1><<<blocks, kThreads, 0, st>>>(W, K, K_prev, s);
  else
    fold_rows_kernel<2><<<blocks, kThreads, 0, st>>>(W, K, K_prev, s);
  return hipGetLastError();
}

}  // namespace awq
