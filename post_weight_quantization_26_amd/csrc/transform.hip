// Steps 3-4 — quantise W·diag(s_c) group-wise, dequantise, fold diag(s_c)^-1
// back and subtract W, for every candidate c of a batch:
//
//   E_c[n][k] = (q - zero)·step / s_c[k] - W[n][k]
//
// so that X·E_cᵀ = Y_c - Y, the output error of candidate c ("05 — AWQ",
// section 3 "The scaling trick" for the fold; section 4 for quantise then
// measure the output error; "Optional: per-channel clipping" for the ratio).
//
// E may hold several layers side by side (linears sharing one input are
// searched together): candidate c of a layer starts `cand_stride` elements
// after candidate c-1, and the caller offsets E to the layer's first row.
//
// One lane owns 8 consecutive input channels of one row; the 16 lanes of a
// 128-wide group find its min/max with xor-shuffles, so every lane holds the
// group's step and zero point. W is read once per batch and each candidate's
// E row segment is written with one 16-byte store per lane.
//
// Arithmetic per element: w' = w·s; the code quotient w'/step comes from the
// group's IEEE reciprocal and one FMA correction (quant_code), as in the
// packed output. The fold multiplies by a precomputed table 1/s instead of
// dividing by s.
//
// Split operands (16-bit types only): each float32 e is stored as two
// halves hi = rnd(e), lo = rnd(e - hi), both round-to-nearest-even, so hi +
// lo is e to ~16 significand bits. A row then has length 2K with the halves
// in alternating 128-wide blocks: channel k's hi at (k / 128)·256 + k % 128,
// its lo 128 further on (the layout the search GEMM's split kernels read).
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;

template <int DT>
__device__ __forceinline__ void store8(void* E, int64_t idx, const float (&e)[8]);
template <int DT>
__device__ __forceinline__ float rounded(float e);
template <>
__device__ __forceinline__ float rounded<1>(float e) {
  return float(static_cast<__bf16>(e));
}
template <>
__device__ __forceinline__ float rounded<2>(float e) {
  return float(static_cast<_Float16>(e));
}

// bf16 output: gfx950 converts float32 to bf16 in hardware with round-to-nearest-even.
template <>
__device__ __forceinline__ void store8<1>(void* E, int64_t idx, const float (&e)[8]) {
  uint16_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(e[i]));
  uint4 q;
  q.x = uint32_t(h[0]) | (uint32_t(h[1]) << 16);
  q.y = uint32_t(h[2]) | (uint32_t(h[3]) << 16);
  q.z = uint32_t(h[4]) | (uint32_t(h[5]) << 16);
  q.w = uint32_t(h[6]) | (uint32_t(h[7]) << 16);
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(E) + idx) = q;
}

// fp16 output: hardware conversion, round-to-nearest-even (subnormals kept).
template <>
__device__ __forceinline__ void store8<2>(void* E, int64_t idx, const float (&e)[8]) {
  uint16_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(e[i]));
  uint4 q;
  q.x = uint32_t(h[0]) | (uint32_t(h[1]) << 16);
  q.y = uint32_t(h[2]) | (uint32_t(h[3]) << 16);
  q.z = uint32_t(h[4]) | (uint32_t(h[5]) << 16);
  q.w = uint32_t(h[6]) | (uint32_t(h[7]) << 16);
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(E) + idx) = q;
}

template <>
__device__ __forceinline__ void store8<0>(void* E, int64_t idx, const float (&e)[8]) {
  float4* p = reinterpret_cast<float4*>(static_cast<float*>(E) + idx);
  p[0] = make_float4(e[0], e[1], e[2], e[3]);
  p[1] = make_float4(e[4], e[5], e[6], e[7]);
}

// DT: 0 = f32 (E in f32), 1 = bf16 (E in bf16), 2 = fp16 (E in fp16). G:
// group size (32, 64, 128);
// the G/8 lanes of a group reduce its range. SPLIT (DT 1 or 2): hi/lo rows.
template <int DT, int G, bool SPLIT>
__global__ __launch_bounds__(kThreads) void transform_kernel(
    const void* __restrict__ W, int64_t N, int64_t K, const float* __restrict__ s_rows,
    const float* __restrict__ inv_rows, int64_t s_stride, GridArgs ratios, int has_ratio, int nc,
    int bits, int zero_point, void* __restrict__ E, int64_t cand_stride) {
#pragma clang fp contract(off)
  const int64_t NK = N * K;
  const int64_t e0 = (int64_t(blockIdx.x) * kThreads + threadIdx.x) * 8;  // flat n*K + k
  // NK is a multiple of 128, so the lanes of a group are all in range or all out.
  const bool active = e0 < NK;
  const int64_t k = active ? e0 % K : 0;

  float w[8];
  if (active) {
    load8<DT>(W, e0, w);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0.f;
  }

  for (int c = 0; c < nc; ++c) {
    // 16-byte aligned rows (k is a multiple of 8); idle lanes read column 0.
    const float4* s4 = reinterpret_cast<const float4*>(s_rows + int64_t(c) * s_stride + k);
    const float4* i4 = reinterpret_cast<const float4*>(inv_rows + int64_t(c) * s_stride + k);
    const float4 sa = s4[0], sb = s4[1], ia = i4[0], ib = i4[1];
    const float sv[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
    const float iv[8] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
    float wp[8];
    float mx = 0.f, mn = 0.f;  // range widened to contain 0
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      wp[i] = w[i] * sv[i];
      mx = fmaxf(mx, wp[i]);
      mn = fminf(mn, wp[i]);
    }
#pragma unroll
    for (int off = 1; off < G / 8; off <<= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, off));
      mn = fminf(mn, __shfl_xor(mn, off));
    }
    const float r = has_ratio ? ratios.v[c] : 1.f;
    const QParams p = group_qparams(mx, mn, r, bits, zero_point);
    const float rstep = 1.0f / p.step;
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = quant_code(wp[i], p, rstep);
      e[i] = ((q - p.zero) * p.step) * iv[i] - w[i];
    }
    if (!active) continue;
    if (SPLIT) {
      // row n = e0 / K; channel k's 128-block b = k / 128 holds hi at 256·b
      const int64_t o = int64_t(c) * cand_stride + (e0 - k) * 2 + (k >> 7) * 256 + (k & 127);
      float lo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float h = rounded<DT>(e[i]);
        lo[i] = e[i] - h;
        e[i] = h;
      }
      store8<DT>(E, o, e);
      store8<DT>(E, o + 128, lo);
    } else {
      store8<DT>(E, int64_t(c) * cand_stride + e0, e);
    }
  }
}

template <int DT, bool SPLIT>
hipError_t launch_transform_g(int group, unsigned blocks, hipStream_t st, const void* W, int64_t N,
                              int64_t K, const float* s_rows, const float* inv_rows,
                              int64_t s_stride, const GridArgs& g, int has_ratio, int nc,
                              int bits, int zero_point, void* E, int64_t cand_stride) {
  if (group == 32)
    transform_kernel<DT, 32, SPLIT><<<blocks, kThreads, 0, st>>>(
        W, N, K, s_rows, inv_rows, s_stride, g, has_ratio, nc, bits, zero_point, E, cand_stride);
  else if (group == 64)
    transform_kernel<DT, 64, SPLIT><<<blocks, kThreads, 0, st>>>(
        W, N, K, s_rows, inv_rows, s_stride, g, has_ratio, nc, bits, zero_point, E, cand_stride);
  else
    transform_kernel<DT, 128, SPLIT><<<blocks, kThreads, 0, st>>>(
        W, N, K, s_rows, inv_rows, s_stride, g, has_ratio, nc, bits, zero_point, E, cand_stride);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_transform(const void* W, int dtype, int64_t N, int64_t K, const float* s_rows,
                            const float* inv_rows, int64_t s_stride, const float* ratios_host,
                            int nc, int bits, int group, int zero_point, int split, void* E,
                            int64_t cand_stride, hipStream_t st) {
  GridArgs g{};
  const int has_ratio = ratios_host != nullptr;
  for (int i = 0; i < nc && i < 64; ++i) g.v[i] = has_ratio ? ratios_host[i] : 1.f;
  const int64_t lanes = N * K / 8;
  const unsigned blocks = unsigned((lanes + kThreads - 1) / kThreads);
  if (dtype == 1 && split)
    return launch_transform_g<1, true>(group, blocks, st, W, N, K, s_rows, inv_rows, s_stride, g,
                                       has_ratio, nc, bits, zero_point, E, cand_stride);
  if (dtype == 1)
    return launch_transform_g<1, false>(group, blocks, st, W, N, K, s_rows, inv_rows, s_stride, g,
                                        has_ratio, nc, bits, zero_point, E, cand_stride);
  if (dtype == 2 && split)
    return launch_transform_g<2, true>(group, blocks, st, W, N, K, s_rows, inv_rows, s_stride, g,
                                       has_ratio, nc, bits, zero_point, E, cand_stride);
  if (dtype == 2)
    return launch_transform_g<2, false>(group, blocks, st, W, N, K, s_rows, inv_rows, s_stride, g,
                                        has_ratio, nc, bits, zero_point, E, cand_stride);
  return launch_transform_g<0, false>(group, blocks, st, W, N, K, s_rows, inv_rows, s_stride, g,
                                      has_ratio, nc, bits, zero_point, E, cand_stride);
}

}  // namespace awq
