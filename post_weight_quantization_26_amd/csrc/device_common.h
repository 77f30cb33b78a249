// Device-side helpers shared by the HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

// Kernel launchers, implemented next to their kernels. Each returns the HIP
// status of the launch.
hipError_t launch_stats(const void* X, int dtype, int64_t T, int64_t K, int64_t chunks,
                        double* partial, float* abar, hipStream_t st);
hipError_t launch_scale_table(const float* abar, int64_t K, const float* alphas_host, int n,
                              float* s_table, float* inv_table, hipStream_t st);
hipError_t launch_reciprocal(const float* s, int64_t n, float* s_copy, float* inv,
                             hipStream_t st);
// Candidate error weights E[c] = fold(dequant(quant(W·diag(s_c), r_c))) - W for
// c in [0, nc): scale rows `s_rows` (s_stride 0 = one shared row) and clip
// ratios `ratios_host` (NULL = all 1). Candidate c's [N, K] block starts at
// element c·cand_stride of E. split (16-bit types): rows of 2K elements, hi
// and lo halves in alternating 128-wide blocks.
hipError_t launch_transform(const void* W, int dtype, int64_t N, int64_t K, const float* s_rows,
                            const float* inv_rows, int64_t s_stride, const float* ratios_host,
                            int nc, int bits, int group, int zero_point, int split, void* E,
                            int64_t cand_stride, hipStream_t st);
// In-place fold of 1/s: v[j] /= s[j] (j < K); rows of W [K, K_prev] /= s[row].
hipError_t launch_fold_vec(void* v, int dtype, int64_t K, const float* s, hipStream_t st);
hipError_t launch_fold_rows(void* W, int dtype, int64_t K, int64_t K_prev, const float* s,
                            hipStream_t st);
// partials[mt][c] = Σ_{t in tile mt} (X·Eᵀ)[t][c]² for c in [0, Nc); with
// split, E rows are hi/lo halves (2K elements) and the product is X·(hi+lo)ᵀ.
hipError_t launch_search_gemm(const void* X, int dtype, const void* E, int64_t M, int64_t Nc,
                              int64_t K, int split, float* partials, hipStream_t st);
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

// Grid values travel to kernels by value.
struct GridArgs {
  float v[64];
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, h);
  return float(v);
}

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Load 8 consecutive elements starting at p (16-byte aligned for 2-byte
// types, 32 bytes for f32) as float32.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<1>(const void* base, int64_t idx, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load8<2>(const void* base, int64_t idx, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = f16_to_f32(uint16_t(w[i] & 0xFFFFu));
    v[2 * i + 1] = f16_to_f32(uint16_t(w[i] >> 16));
  }
}

template <>
__device__ __forceinline__ void load8<0>(const void* base, int64_t idx, float (&v)[8]) {
  const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
  const float4 a = p[0], b = p[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Group quantiser parameters from the group's (0-widened) range, IEEE f32.
// mx >= 0 >= mn are the group max/min of w' already widened to contain 0.
struct QParams {
  float step;
  float zero;
  float qmax;
};

__device__ __forceinline__ QParams group_qparams(float mx, float mn, float ratio, int bits,
                                                 int zero_point) {
#pragma clang fp contract(off)
  QParams p;
  p.qmax = float((1 << bits) - 1);
  mx = ratio * mx;
  mn = ratio * mn;
  if (zero_point) {
    p.step = fmaxf((mx - mn) / p.qmax, 1e-5f);
    p.zero = fminf(fmaxf(__builtin_rintf(-mn / p.step), 0.f), p.qmax);
  } else {
    const float amax = fmaxf(mx, -mn);
    p.step = fmaxf(amax / float((1 << (bits - 1)) - 1), 1e-5f);
    p.zero = float(1 << (bits - 1));
  }
  return p;
}

// Code of a scaled weight, less its zero point: q - zero with q =
// clamp(rint(w'/step) + zero, 0, qmax). The quotient w'/step comes from the
// group's IEEE reciprocal `rstep` = 1/step and one FMA correction step, which
// gives the correctly rounded quotient up to at most one ulp in rare cases; a
// code can differ from exact division only when the quotient lies within one
// ulp of a .5 rounding boundary. rint(quotient), zero and qmax are integers
// held exactly in float32, so clamping rint(quotient) to [-zero, qmax - zero]
// (one med3) is the clamp of the code and the subtraction of the zero point.
__device__ __forceinline__ float quant_code_centered(float wp, const QParams& p, float rstep) {
  const float q0 = wp * rstep;
  const float quo = __builtin_fmaf(__builtin_fmaf(-q0, p.step, wp), rstep, q0);
  return __builtin_amdgcn_fmed3f(__builtin_rintf(quo), -p.zero, p.qmax - p.zero);
}

}  // namespace awq
