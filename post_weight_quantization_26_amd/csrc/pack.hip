// Step 8 — quantise W·diag(s) (row n clipped by ratio[n]) to 4-bit codes and
// pack them in the AWQ storage layout ("05 — AWQ", section 5 "Bit-level
// output format"):
//
//   qweight [K, N/8] int32   word (k, j): rows 8j..8j+7 at column k, row 8j+i in bits 4i..
//   qzeros  [K/128, N/8]     the groups' zero points, packed the same way
//   scales  [K/128, N] fp16  the groups' steps (RNE of the float32 step)
//
// A workgroup owns 256 output rows x one 128-channel group. Lane (c, jb)
// reads 8 consecutive channels of 8 consecutive rows (16 lanes cover a row's
// group: 256 contiguous bytes per row for bf16), finds each row's group
// range with xor-shuffles over those 16 lanes, and packs its 8x8 codes into 8
// words in registers. Words are transposed through LDS so every qweight row
// segment is written with consecutive 4-byte stores. One pass over W: HBM
// bound. Codes: IEEE float32 group parameters, quotient from the group's
// reciprocal with one FMA correction, rint.
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 256;

template <int DT>
__global__ __launch_bounds__(kThreads) void pack_kernel(
    const void* __restrict__ W, int64_t N, int64_t K, const float* __restrict__ s,
    const float* __restrict__ ratio, int zero_point, int32_t* __restrict__ qweight,
    int32_t* __restrict__ qzeros, uint16_t* __restrict__ scales, int* __restrict__ overflow) {
#pragma clang fp contract(off)
  __shared__ uint32_t words[128][33];
  __shared__ uint16_t sc_lds[kRows];
  __shared__ uint8_t z_lds[kRows];

  const int tid = threadIdx.x;
  const int c = tid & 15, jb = tid >> 4;
  const int64_t n0 = int64_t(blockIdx.x) * kRows;
  const int64_t g = blockIdx.y;
  const int64_t k = g * 128 + c * 8;
  const int64_t N8 = N / 8;

  float sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = s[k + i];

#pragma unroll 1
  for (int u = 0; u < 2; ++u) {
    const int j = jb + 16 * u;
    uint32_t wd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 1
    for (int r8 = 0; r8 < 8; ++r8) {
      const int row = 8 * j + r8;
      const int64_t n = n0 + row;
      const bool valid = n < N;
      float w[8];
      if (valid) {
        load8<DT>(W, n * K + k, w);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = 0.f;
      }
      float wp[8], mx = 0.f, mn = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        wp[i] = w[i] * sv[i];
        mx = fmaxf(mx, wp[i]);
        mn = fminf(mn, wp[i]);
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        mx = fmaxf(mx, __shfl_xor(mx, off));
        mn = fminf(mn, __shfl_xor(mn, off));
      }
      const float r = (ratio != nullptr && valid) ? ratio[n] : 1.f;
      const QParams p = group_qparams(mx, mn, r, 4, zero_point);
      const float rstep = 1.0f / p.step;
#pragma unroll
      for (int i = 0; i < 8; ++i) wd[i] |= uint32_t(quant_code(wp[i], p, rstep)) << (4 * r8);
      if (c == 0) {
        const _Float16 h = _Float16(p.step);
        const uint16_t hb = __builtin_bit_cast(uint16_t, h);
        sc_lds[row] = hb;
        z_lds[row] = uint8_t(p.zero);
        if (valid && (hb & 0x7FFFu) >= 0x7C00u) *overflow = 1;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) words[c * 8 + i][j] = wd[i];
  }
  __syncthreads();

  const int jj = tid & 31;
  const int64_t jcol = n0 / 8 + jj;
  if (jcol < N8) {
#pragma unroll 4
    for (int v = 0; v < 16; ++v) {
      const int kk = (tid >> 5) + 8 * v;
      qweight[(g * 128 + kk) * N8 + jcol] = int32_t(words[kk][jj]);
    }
  }
  if (n0 + tid < N) scales[g * N + n0 + tid] = sc_lds[tid];
  if (tid < 32 && n0 / 8 + tid < N8) {
    uint32_t zw = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) zw |= uint32_t(z_lds[8 * tid + i]) << (4 * i);
    qzeros[g * N8 + n0 / 8 + tid] = int32_t(zw);
  }
}

}  // namespace

hipError_t launch_pack(const void* W, int dtype, int64_t N, int64_t K, const float* s,
                       const float* ratio, int zero_point, int32_t* qweight, int32_t* qzeros,
                       uint16_t* scales, int* overflow, hipStream_t st) {
  dim3 grid(unsigned((N + kRows - 1) / kRows), unsigned(K / 128));
  if (dtype == 1)
    pack_kernel<1><<<grid, kThreads, 0, st>>>(W, N, K, s, ratio, zero_point, qweight, qzeros,
                                              scales, overflow);
  else if (dtype == 2)
    pack_kernel<2><<<grid, kThreads, 0, st>>>(W, N, K, s, ratio, zero_point, qweight, qzeros,
                                              scales, overflow);
  else
    pack_kernel<0><<<grid, kThreads, 0, st>>>(W, N, K, s, ratio, zero_point, qweight, qzeros,
                                              scales, overflow);
  return hipGetLastError();
}

}  // namespace awq
