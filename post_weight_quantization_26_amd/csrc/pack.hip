// Step 8 — quantise W·diag(s) (row n clipped by ratio[n]) to b-bit codes
// (b = 4 or 3) and pack them in the AWQ storage layout ("05 — AWQ", section 5
// "Bit-level output format"):
//
//   qweight [K, N·b/32] int32   codes of column k packed along the output dim
//   qzeros  [K/g, N·b/32]       the groups' zero points, packed the same way
//   scales  [K/g, N] fp16       the groups' steps (RNE of the float32 step)
//
// Packing is dense from the lowest bit up: row n's code sits at bits
// b·n .. b·n + b - 1 of the little-endian stream of a qweight row. For 4 bits
// that is 8 codes per word, row 8j+i in bits 4i..4i+3 of word j (the page's
// layout); for 3 bits 32 rows fill 3 words and some codes straddle two.
//
// A workgroup owns 256 output rows x one 128-channel tile of the input dim
// (1, 2 or 4 groups of g = 128, 64 or 32 channels). Lane (c, jb) reads 8
// consecutive channels of 8 consecutive rows, finds each row's group range
// with xor-shuffles over the g/8 lanes of its group, and packs the 8 codes of
// each of its channels into the low 8·b bits of a word in registers. Those
// partial words are transposed through LDS: for 4 bits each is one qweight
// word; for 3 bits four of them (32 rows) make three words. qweight rows are
// written with consecutive stores. One pass over W. Codes: IEEE float32 group
// parameters, quotient from the group's reciprocal with one FMA correction,
// rint.
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 256;
constexpr int kTile = 128;   // input channels per workgroup

template <int DT, int BITS, int G>
__global__ __launch_bounds__(kThreads) void pack_kernel(
    const void* __restrict__ W, int64_t N, int64_t K, const float* __restrict__ s,
    const float* __restrict__ ratio, int zero_point, int32_t* __restrict__ qweight,
    int32_t* __restrict__ qzeros, uint16_t* __restrict__ scales, int* __restrict__ overflow) {
#pragma clang fp contract(off)
  constexpr int kGroups = kTile / G;     // groups per tile
  constexpr int kLanes = G / 8;          // lanes per group
  __shared__ uint32_t words[kTile][33];
  __shared__ uint16_t sc_lds[kGroups][kRows];
  __shared__ uint8_t z_lds[kGroups][kRows];

  const int tid = threadIdx.x;
  const int c = tid & 15, jb = tid >> 4;
  const int gi = c / kLanes;                       // this lane's group within the tile
  const int64_t n0 = int64_t(blockIdx.x) * kRows;
  const int64_t tile = blockIdx.y;
  const int64_t k = tile * kTile + c * 8;

  float sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = s[k + i];

#pragma unroll 1
  for (int u = 0; u < 2; ++u) {
    const int j = jb + 16 * u;                     // 8-row chunk, 0..31
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
      for (int off = 1; off < kLanes; off <<= 1) {
        mx = fmaxf(mx, __shfl_xor(mx, off));
        mn = fminf(mn, __shfl_xor(mn, off));
      }
      const float r = (ratio != nullptr && valid) ? ratio[n] : 1.f;
      const QParams p = group_qparams(mx, mn, r, BITS, zero_point);
      const float rstep = 1.0f / p.step;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        wd[i] |= uint32_t(quant_code(wp[i], p, rstep)) << (BITS * r8);
      if (c % kLanes == 0) {
        const _Float16 h = _Float16(p.step);
        const uint16_t hb = __builtin_bit_cast(uint16_t, h);
        sc_lds[gi][row] = hb;
        z_lds[gi][row] = uint8_t(p.zero);
        if (valid && (hb & 0x7FFFu) >= 0x7C00u) *overflow = 1;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) words[c * 8 + i][j] = wd[i];
  }
  __syncthreads();

  const int64_t g0 = tile * kGroups;               // first group row of this tile
  if constexpr (BITS == 4) {
    const int64_t N8 = N / 8;
    const int jj = tid & 31;
    const int64_t jcol = n0 / 8 + jj;
    if (jcol < N8) {
#pragma unroll 4
      for (int v = 0; v < 16; ++v) {
        const int kk = (tid >> 5) + 8 * v;
        qweight[(tile * kTile + kk) * N8 + jcol] = int32_t(words[kk][jj]);
      }
    }
    const int zg = tid >> 5;
    if (zg < kGroups && jcol < N8) {
      uint32_t zw = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) zw |= uint32_t(z_lds[zg][8 * jj + i]) << (4 * i);
      qzeros[(g0 + zg) * N8 + jcol] = int32_t(zw);
    }
  } else {
    // 3 bits: four 24-bit partial words (rows 32q .. 32q+31) -> three words.
    const int64_t N32 = N / 32, N3 = N32 * 3;
    const int q = tid & 7;
    const int64_t qcol = n0 / 32 + q;
    if (qcol < N32) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int kk = (tid >> 3) + 32 * v;
        const uint32_t a = words[kk][4 * q], b = words[kk][4 * q + 1];
        const uint32_t cc = words[kk][4 * q + 2], d = words[kk][4 * q + 3];
        int32_t* dst = qweight + (tile * kTile + kk) * N3 + 3 * qcol;
        dst[0] = int32_t(a | (b << 24));
        dst[1] = int32_t((b >> 8) | (cc << 16));
        dst[2] = int32_t((cc >> 16) | (d << 8));
      }
    }
    const int zg = tid >> 3;
    if (zg < kGroups && qcol < N32) {
      uint32_t z3[3] = {0, 0, 0};
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t z = z_lds[zg][32 * q + i];
        const int bit = 3 * i, w = bit >> 5, sh = bit & 31;
        z3[w] |= z << sh;
        if (sh > 29) z3[w + 1] |= z >> (32 - sh);
      }
      int32_t* dst = qzeros + (g0 + zg) * N3 + 3 * qcol;
      dst[0] = int32_t(z3[0]);
      dst[1] = int32_t(z3[1]);
      dst[2] = int32_t(z3[2]);
    }
  }
#pragma unroll
  for (int zg = 0; zg < kGroups; ++zg)
    if (n0 + tid < N) scales[(g0 + zg) * N + n0 + tid] = sc_lds[zg][tid];
}

template <int DT, int BITS>
hipError_t launch_pack_g(int group, dim3 grid, hipStream_t st, const void* W, int64_t N,
                         int64_t K, const float* s, const float* ratio, int zero_point,
                         int32_t* qweight, int32_t* qzeros, uint16_t* scales, int* overflow) {
  if (group == 32)
    pack_kernel<DT, BITS, 32><<<grid, kThreads, 0, st>>>(W, N, K, s, ratio, zero_point, qweight,
                                                         qzeros, scales, overflow);
  else if (group == 64)
    pack_kernel<DT, BITS, 64><<<grid, kThreads, 0, st>>>(W, N, K, s, ratio, zero_point, qweight,
                                                         qzeros, scales, overflow);
  else
    pack_kernel<DT, BITS, 128><<<grid, kThreads, 0, st>>>(W, N, K, s, ratio, zero_point, qweight,
                                                          qzeros, scales, overflow);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_pack_b(int bits, int group, dim3 grid, hipStream_t st, const void* W,
                         int64_t N, int64_t K, const float* s, const float* ratio, int zero_point,
                         int32_t* qweight, int32_t* qzeros, uint16_t* scales, int* overflow) {
  if (bits == 3)
    return launch_pack_g<DT, 3>(group, grid, st, W, N, K, s, ratio, zero_point, qweight, qzeros,
                                scales, overflow);
  return launch_pack_g<DT, 4>(group, grid, st, W, N, K, s, ratio, zero_point, qweight, qzeros,
                              scales, overflow);
}

}  // namespace

hipError_t launch_pack(const void* W, int dtype, int64_t N, int64_t K, const float* s,
                       const float* ratio, int bits, int group, int zero_point, int32_t* qweight,
                       int32_t* qzeros, uint16_t* scales, int* overflow, hipStream_t st) {
  dim3 grid(unsigned((N + kRows - 1) / kRows), unsigned(K / kTile));
  if (dtype == 1)
    return launch_pack_b<1>(bits, group, grid, st, W, N, K, s, ratio, zero_point, qweight, qzeros,
                            scales, overflow);
  if (dtype == 2)
    return launch_pack_b<2>(bits, group, grid, st, W, N, K, s, ratio, zero_point, qweight, qzeros,
                            scales, overflow);
  return launch_pack_b<0>(bits, group, grid, st, W, N, K, s, ratio, zero_point, qweight, qzeros,
                          scales, overflow);
}

}  // namespace awq
