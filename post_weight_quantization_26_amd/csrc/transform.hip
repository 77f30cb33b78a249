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
// One lane owns 8 consecutive input channels of 4 consecutive rows; the 16
// lanes of a 128-wide group find its min/max with DPP steps. W is read once
// per batch and each candidate's E row segment is written with one 16-byte
// store per lane and row.
//
// Arithmetic per element: w' = w·s; the code quotient w'/step comes from the
// group's IEEE reciprocal and one FMA correction (quant_code_centered, which
// also clamps the code and takes off the zero point in one med3), as in the
// packed output. The fold multiplies by a precomputed table 1/s instead of
// dividing by s. A group's step, zero point and reciprocal are formed by one
// lane per candidate and shared by DPP broadcasts.
//
// Split operands (16-bit types only): each float32 e is stored as two
// halves hi = rnd(e), lo = rnd(e - hi), both round-to-nearest-even, so hi +
// lo is e to ~16 significand bits. A row then has length 2K with the halves
// in alternating 128-wide blocks: channel k's hi at (k / 128)·256 + k % 128,
// its lo 128 further on (the layout the search GEMM's split kernels read).
#include <utility>

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

// Cross-lane moves inside a group of L = 4, 8 or 16 lanes (aligned runs of
// a 16-lane DPP row), as VALU instructions instead of LDS round trips. Every
// lane's source lies in its own row, so no lane reads out of range.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// One reduction step, max or min of v and v from lane l ^ 1 (quad_perm
// [1, 0, 3, 2]), l ^ 2 ([2, 3, 0, 1]), 7 - l within each half row
// (row_half_mirror) or 15 - l within the row (row_mirror), as one
// DPP-modified v_max_f32 / v_min_f32. Written out because the compiler puts
// a NaN-quieting max after every DPP move it cannot see through (the values
// here are products of finite floats); the s_nop covers the two wait states
// a DPP read needs after the VALU write of its source.
#define AWQ_DPP_STEP(NAME, OP, CTRLSTR)                                                       \
  __device__ __forceinline__ float NAME(float v) {                                           \
    float r;                                                                                  \
    asm("s_nop 1\n\t" OP " %0, %1, %1 " CTRLSTR " row_mask:0xf bank_mask:0xf"              \
        : "=v"(r) : "v"(v));                                                                  \
    return r;                                                                                 \
  }
AWQ_DPP_STEP(max_x1, "v_max_f32_dpp", "quad_perm:[1,0,3,2]")
AWQ_DPP_STEP(max_x2, "v_max_f32_dpp", "quad_perm:[2,3,0,1]")
AWQ_DPP_STEP(max_hm, "v_max_f32_dpp", "row_half_mirror")
AWQ_DPP_STEP(max_rm, "v_max_f32_dpp", "row_mirror")
AWQ_DPP_STEP(min_x1, "v_min_f32_dpp", "quad_perm:[1,0,3,2]")
AWQ_DPP_STEP(min_x2, "v_min_f32_dpp", "quad_perm:[2,3,0,1]")
AWQ_DPP_STEP(min_hm, "v_min_f32_dpp", "row_half_mirror")
AWQ_DPP_STEP(min_rm, "v_min_f32_dpp", "row_mirror")
#undef AWQ_DPP_STEP
// every lane of the group gets the group's max (MAX) or min: lanes xor 1 and
// xor 2 within a quad, then the half-row mirror (lane i and 7 - i: the other
// quad of 8 lanes), then the row mirror (lane i and 15 - i: the other half)
template <int L, bool MAX>
__device__ __forceinline__ float group_reduce(float v) {
  v = MAX ? max_x1(v) : min_x1(v);
  v = MAX ? max_x2(v) : min_x2(v);
  if constexpr (L >= 8) v = MAX ? max_hm(v) : min_hm(v);
  if constexpr (L >= 16) v = MAX ? max_rm(v) : min_rm(v);
  return v;
}
// lane I of the group, for every lane of the group
template <int L, int I>
__device__ __forceinline__ float group_bcast(float v) {
  if constexpr (L == 16) {
    return dpp<0x150 + I>(v);                 // row_newbcast: lane I of the row
  } else if constexpr (L == 8) {
    const float a = dpp<0x150 + I>(v), b = dpp<0x158 + I>(v);
    return (threadIdx.x & 8) ? b : a;
  } else {
    return dpp<I | (I << 2) | (I << 4) | (I << 6)>(v);   // quad_perm [I, I, I, I]
  }
}

// f(integral_constant<I>) for I = 0 .. n - 1 (n <= the sequence's length)
template <class F, int... Is>
__device__ __forceinline__ void first_n(F& f, int n, std::integer_sequence<int, Is...>) {
  ((Is < n ? f(std::integral_constant<int, Is>{}) : void()), ...);
}

// 8 consecutive float32 scale (or reciprocal) entries of candidate row c
__device__ __forceinline__ void load_row8(const float* rows, int64_t stride, int c, int64_t k,
                                          float (&v)[8]) {
  // 16-byte aligned rows (k is a multiple of 8)
  const float4* p = reinterpret_cast<const float4*>(rows + int64_t(c) * stride + k);
  const float4 a = p[0], b = p[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// DT: 0 = f32 (E in f32), 1 = bf16 (E in bf16), 2 = fp16 (E in fp16). G:
// group size (32, 64, 128); the L = G/8 lanes of a group reduce its range.
// SPLIT (DT 1 or 2): hi/lo rows. PARAMS: instead of E, write each (candidate,
// row, group)'s {step, zero, 1/step, 0} to E as float4, entry
// c·cand_stride + n·(K/G) + k/G. R: rows per lane.
//
// A lane owns 8 consecutive channels of R consecutive rows: the candidates'
// scale and reciprocal entries of those channels, which every row needs, are
// loaded once for the R rows (they come from L2, and per element they would
// otherwise be three times the bytes of W and E together).
//
// The candidates go in chunks of L: first every lane forms the group ranges
// of the chunk's candidates (DPP reductions over the group's lanes), and lane
// i of the group keeps candidate i's; then each lane forms the step and zero
// point of its own candidate (the IEEE divisions, once per group and
// candidate instead of once per lane); then, candidate by candidate, the
// group's lanes take them from lane i by DPP broadcast and quantise their 8
// channels.
template <int DT, int G, bool SPLIT, bool PARAMS, int R>
__global__ __launch_bounds__(kThreads) void transform_kernel(
    const void* __restrict__ W, int64_t N, int64_t K, const float* __restrict__ s_rows,
    const float* __restrict__ inv_rows, int64_t s_stride, GridArgs ratios, int has_ratio, int nc,
    int bits, int zero_point, void* __restrict__ E, int64_t cand_stride) {
#pragma clang fp contract(off)
  constexpr int L = G / 8;
  const int64_t K8 = K / 8;
  const int64_t lid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  // rows R·rb .. R·rb + R - 1, channels k .. k + 7. K is a multiple of 128,
  // so the lanes of a group share their rows: all in range or all out.
  const int64_t rb = lid / K8;
  const int64_t k = (lid - rb * K8) * 8;
  const int64_t n0 = rb * R;
  const int lig = threadIdx.x & (L - 1);                 // lane within the group

  bool act[R];
  float w[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    act[r] = n0 + r < N;
    if (act[r]) {
      load8<DT>(W, (n0 + r) * K + k, w[r]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[r][i] = 0.f;
    }
  }

  for (int c0 = 0; c0 < nc; c0 += L) {
    const int nl = nc - c0 < L ? nc - c0 : L;
    // ranges of the chunk's candidates; lane i of the group keeps candidate c0 + i's
    float kmx[R], kmn[R];
#pragma unroll
    for (int r = 0; r < R; ++r) kmx[r] = kmn[r] = 0.f;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if (i < nl) {   // the same for every lane
        float sv[8];
        load_row8(s_rows, s_stride, c0 + i, k, sv);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float mx = 0.f, mn = 0.f;  // range widened to contain 0
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float wp = w[r][t] * sv[t];
            mx = fmaxf(mx, wp);
            mn = fminf(mn, wp);
          }
          mx = group_reduce<L, true>(mx);
          mn = group_reduce<L, false>(mn);
          kmx[r] = lig == i ? mx : kmx[r];
          kmn[r] = lig == i ? mn : kmn[r];
        }
      }
    }
    // this lane's candidate: step, zero point and reciprocal of each row
    const int cl = c0 + (lig < nl ? lig : 0);
    const float rr = has_ratio ? ratios.v[cl] : 1.f;
    QParams p[R];
    float rstep[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      p[r] = group_qparams(kmx[r], kmn[r], rr, bits, zero_point);
      rstep[r] = 1.0f / p[r].step;
    }
    if constexpr (PARAMS) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (act[r] && lig < nl)
          reinterpret_cast<float4*>(E)[int64_t(cl) * cand_stride + (n0 + r) * (K / G) + k / G] =
              make_float4(p[r].step, p[r].zero, rstep[r], 0.f);
      }
    } else {
      auto one = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int c = c0 + i;
        float sv[8], iv[8];
        load_row8(s_rows, s_stride, c, k, sv);
        load_row8(inv_rows, s_stride, c, k, iv);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const QParams pc{group_bcast<L, i>(p[r].step), group_bcast<L, i>(p[r].zero), p[r].qmax};
          const float rc = group_bcast<L, i>(rstep[r]);
          float e[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float qc = quant_code_centered(w[r][t] * sv[t], pc, rc);
            e[t] = (qc * pc.step) * iv[t] - w[r][t];
          }
          if (!act[r]) continue;
          const int64_t n = n0 + r;
          if constexpr (SPLIT) {
            // channel k's 128-block b = k / 128 holds hi at 256·b of row n
            const int64_t o = int64_t(c) * cand_stride + n * K * 2 + (k >> 7) * 256 + (k & 127);
            float lo[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const float h = rounded<DT>(e[t]);
              lo[t] = e[t] - h;
              e[t] = h;
            }
            store8<DT>(E, o, e);
            store8<DT>(E, o + 128, lo);
          } else {
            store8<DT>(E, int64_t(c) * cand_stride + n * K + k, e);
          }
        }
      };
      // candidates c0 .. c0 + nl - 1, each with its lane's parameters
      first_n(one, nl, std::make_integer_sequence<int, L>{});
    }
  }
}

// Rows per lane: on the 4096x4096 layer with 20 candidates, 1 / 2 / 4 rows
// took 234 / 188 / 178 us (4 rows: 96-103 VGPRs, 4 waves per SIMD).
constexpr int kRowsPerLane = 4;

template <int DT, bool SPLIT, bool PARAMS>
hipError_t launch_transform_g(int group, hipStream_t st, const void* W, int64_t N,
                              int64_t K, const float* s_rows, const float* inv_rows,
                              int64_t s_stride, const GridArgs& g, int has_ratio, int nc,
                              int bits, int zero_point, void* E, int64_t cand_stride) {
  constexpr int R = kRowsPerLane;
  const int64_t lanes = (N + R - 1) / R * (K / 8);
  const unsigned blocks = unsigned((lanes + kThreads - 1) / kThreads);
  if (group == 32)
    transform_kernel<DT, 32, SPLIT, PARAMS, R><<<blocks, kThreads, 0, st>>>(
        W, N, K, s_rows, inv_rows, s_stride, g, has_ratio, nc, bits, zero_point, E, cand_stride);
  else if (group == 64)
    transform_kernel<DT, 64, SPLIT, PARAMS, R><<<blocks, kThreads, 0, st>>>(
        W, N, K, s_rows, inv_rows, s_stride, g, has_ratio, nc, bits, zero_point, E, cand_stride);
  else
    transform_kernel<DT, 128, SPLIT, PARAMS, R><<<blocks, kThreads, 0, st>>>(
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
  if (dtype == 1 && split)
    return launch_transform_g<1, true, false>(group, st, W, N, K, s_rows, inv_rows,
                                              s_stride, g, has_ratio, nc, bits, zero_point, E,
                                              cand_stride);
  if (dtype == 1)
    return launch_transform_g<1, false, false>(group, st, W, N, K, s_rows, inv_rows,
                                               s_stride, g, has_ratio, nc, bits, zero_point, E,
                                               cand_stride);
  if (dtype == 2 && split)
    return launch_transform_g<2, true, false>(group, st, W, N, K, s_rows, inv_rows,
                                              s_stride, g, has_ratio, nc, bits, zero_point, E,
                                              cand_stride);
  if (dtype == 2)
    return launch_transform_g<2, false, false>(group, st, W, N, K, s_rows, inv_rows,
                                               s_stride, g, has_ratio, nc, bits, zero_point, E,
                                               cand_stride);
  return launch_transform_g<0, false, false>(group, st, W, N, K, s_rows, inv_rows,
                                             s_stride, g, has_ratio, nc, bits, zero_point, E,
                                             cand_stride);
}

// The group parameters of every (candidate, row, group) as float4 {step,
// zero, 1/step, 0}: candidate c's N·K/G entries start c·cand_stride entries
// into P (the fused search's table).
hipError_t launch_group_params(const void* W, int dtype, int64_t N, int64_t K,
                               const float* s_rows, int64_t s_stride, const float* ratios_host,
                               int nc, int bits, int group, int zero_point, float* P,
                               int64_t cand_stride, hipStream_t st) {
  GridArgs g{};
  const int has_ratio = ratios_host != nullptr;
  for (int i = 0; i < nc && i < 64; ++i) g.v[i] = has_ratio ? ratios_host[i] : 1.f;
  if (dtype == 1)
    return launch_transform_g<1, false, true>(group, st, W, N, K, s_rows, s_rows,
                                              s_stride, g, has_ratio, nc, bits, zero_point, P,
                                              cand_stride);
  if (dtype == 2)
    return launch_transform_g<2, false, true>(group, st, W, N, K, s_rows, s_rows,
                                              s_stride, g, has_ratio, nc, bits, zero_point, P,
                                              cand_stride);
  return hipErrorInvalidValue;
}

}  // namespace awq
