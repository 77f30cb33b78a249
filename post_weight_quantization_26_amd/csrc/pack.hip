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
// (1, 2 or 4 groups of g = 128, 64 or 32 channels); consecutive workgroups
// take consecutive tiles of the same rows. Lane (c, jb) takes 8 consecutive
// channels of two 8-row chunks; 16 lanes cover a row's 128 channels, so
// every load instruction reads whole 256-byte row segments (non-temporal: W
// is read once). All 16 rows' loads of a lane are issued before any is used
// (the kernel is otherwise limited by loads in flight). Per 8-row chunk:
//   1. scaled weights of all 8 rows in registers; each row's group range by
//      xor-shuffles over the g/8 lanes of its group;
//   2. the lanes of a group share the per-row group arithmetic (step, zero
//      point, reciprocal: three IEEE float32 divisions): lane ℓ of the group
//      computes it for rows r ≡ ℓ (mod g/8) and the results are broadcast by
//      shuffles, instead of every lane computing all 8 rows;
//   3. codes (quotient from the reciprocal with one FMA correction, rint,
//      clamp) are packed in float arithmetic that is exact (small integers
//      times powers of two, sums below 2^24): acc = fma(code - zero,
//      base^row, acc), the zero points added once per word; 4-bit words use
//      two 16-bit halves.
// The partial words are transposed through LDS: for 4 bits each is one
// qweight word; for 3 bits four of them (32 rows) make three words. qweight
// rows are written with consecutive stores.
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 256;
constexpr int kTile = 128;   // input channels per workgroup

__device__ __forceinline__ uint4 load_stream16(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// Max / min over the kLanes consecutive lanes of a group (4, 8 or 16 lanes,
// aligned within a row of 16) with DPP lane swaps: quad_perm [1,0,3,2] and
// [2,3,0,1] combine within 4 lanes, row_half_mirror pairs the two quads of 8,
// row_mirror the two halves of 16. Every lane ends with its group's value.
template <int kCtrl>
__device__ __forceinline__ void dpp_range_step(float& mx, float& mn) {
  mx = fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, mx),
                                                                    kCtrl, 0xF, 0xF, true)));
  mn = fminf(mn, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, mn),
                                                                    kCtrl, 0xF, 0xF, true)));
}

template <int kLanes>
__device__ __forceinline__ void group_range(float& mx, float& mn) {
  if constexpr (kLanes >= 2) dpp_range_step<0xB1>(mx, mn);    // quad_perm [1,0,3,2]
  if constexpr (kLanes >= 4) dpp_range_step<0x4E>(mx, mn);    // quad_perm [2,3,0,1]
  if constexpr (kLanes >= 8) dpp_range_step<0x141>(mx, mn);   // row_half_mirror
  if constexpr (kLanes >= 16) dpp_range_step<0x140>(mx, mn);  // row_mirror
}

// Raw 16-byte pieces of 8 consecutive elements (one piece for 16-bit types,
// two for float32) and their conversion to float32.
template <int DT>
struct Raw8 {
  uint4 q[DT == 0 ? 2 : 1];
};

template <int DT>
__device__ __forceinline__ void raw_load(const void* base, int64_t idx, Raw8<DT>& r) {
  if constexpr (DT == 0) {
    const float* p = static_cast<const float*>(base) + idx;
    r.q[0] = load_stream16(p);
    r.q[1] = load_stream16(p + 4);
  } else {
    r.q[0] = load_stream16(static_cast<const uint16_t*>(base) + idx);
  }
}

template <int DT>
__device__ __forceinline__ void raw_to_f32(const Raw8<DT>& r, float (&v)[8]) {
  if constexpr (DT == 0) {
    v[0] = __uint_as_float(r.q[0].x); v[1] = __uint_as_float(r.q[0].y);
    v[2] = __uint_as_float(r.q[0].z); v[3] = __uint_as_float(r.q[0].w);
    v[4] = __uint_as_float(r.q[1].x); v[5] = __uint_as_float(r.q[1].y);
    v[6] = __uint_as_float(r.q[1].z); v[7] = __uint_as_float(r.q[1].w);
  } else {
    const uint32_t w[4] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == 1) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      } else {
        v[2 * i] = f16_to_f32(uint16_t(w[i] & 0xFFFFu));
        v[2 * i + 1] = f16_to_f32(uint16_t(w[i] >> 16));
      }
    }
  }
}

template <int DT, int BITS, int G>
__global__ __launch_bounds__(kThreads) void pack_kernel(
    const void* __restrict__ W, int64_t N, int64_t K, const float* __restrict__ s,
    const float* __restrict__ ratio, int zero_point, int32_t* __restrict__ qweight,
    int32_t* __restrict__ qzeros, uint16_t* __restrict__ scales, int* __restrict__ overflow) {
#pragma clang fp contract(off)
  constexpr int kGroups = kTile / G;     // groups per tile
  constexpr int kLanes = G / 8;          // lanes per group
  constexpr int kHalves = BITS == 4 ? 2 : 1;
  __shared__ uint32_t words[kTile][33];
  __shared__ uint16_t sc_lds[kGroups][kRows];
  __shared__ uint8_t z_lds[kGroups][kRows];

  const int tid = threadIdx.x;
  const int c = tid & 15, jb = tid >> 4;
  const int gi = c / kLanes;                       // this lane's group within the tile
  const int gl = c % kLanes;                       // this lane's index within the group
  const int glane0 = (tid & 48) + gi * kLanes;    // wave lane of the group's first lane
  const int64_t n0 = int64_t(blockIdx.y) * kRows;
  const int64_t tile = blockIdx.x;
  const int64_t k = tile * kTile + c * 8;

  float sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = s[k + i];

  // Every load of both 8-row chunks is issued before any is used.
  Raw8<DT> raw[2][8];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      const int64_t n = n0 + 8 * (jb + 16 * u) + r8;
      if (n < N) {
        raw_load<DT>(W, n * K + k, raw[u][r8]);
      } else {
#pragma unroll
        for (int q = 0; q < (DT == 0 ? 2 : 1); ++q) raw[u][r8].q[q] = make_uint4(0, 0, 0, 0);
      }
    }

#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = jb + 16 * u;                     // 8-row chunk, 0..31
    // 1. scaled weights and each row's 0-widened group range
    float wp[8][8], mx[8], mn[8];
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      float w[8];
      raw_to_f32<DT>(raw[u][r8], w);
      mx[r8] = 0.f;
      mn[r8] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        wp[r8][i] = w[i] * sv[i];
        mx[r8] = fmaxf(mx[r8], wp[r8][i]);
        mn[r8] = fminf(mn[r8], wp[r8][i]);
      }
    }
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) group_range<kLanes>(mx[r8], mn[r8]);
    // 2. group arithmetic of rows r ≡ gl (mod kLanes), then broadcast
    constexpr int kMine = kLanes >= 8 ? 1 : 8 / kLanes;   // rows this lane computes
    float my_step[kMine], my_zero[kMine], my_rstep[kMine];
#pragma unroll
    for (int m = 0; m < kMine; ++m) {
      const int r8 = kLanes >= 8 ? (gl & 7) : gl + kLanes * m;
      float mxr = mx[0], mnr = mn[0];
#pragma unroll
      for (int q = 1; q < 8; ++q)
        if (q == r8) { mxr = mx[q]; mnr = mn[q]; }
      const int64_t n = n0 + 8 * j + r8;
      const bool valid = n < N;
      const float r = (ratio != nullptr && valid) ? ratio[n] : 1.f;
      const QParams p = group_qparams(mxr, mnr, r, BITS, zero_point);
      my_step[m] = p.step;
      my_zero[m] = p.zero;
      my_rstep[m] = 1.0f / p.step;
      if (gl == r8 % kLanes && gl < 8) {
        const _Float16 hf = _Float16(p.step);
        const uint16_t hb = __builtin_bit_cast(uint16_t, hf);
        sc_lds[gi][8 * j + r8] = hb;
        z_lds[gi][8 * j + r8] = uint8_t(p.zero);
        if (valid && (hb & 0x7FFFu) >= 0x7C00u) *overflow = 1;
      }
    }
    // 3. codes, packed exactly in float
    const float qmax = float((1 << BITS) - 1);
    float acc[kHalves][8], zacc[kHalves];
#pragma unroll
    for (int h = 0; h < kHalves; ++h) {
      zacc[h] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
    }
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      const int src = glane0 + (r8 % kLanes);
      const int m = kLanes >= 8 ? 0 : r8 / kLanes;
      const float step = __shfl(my_step[m], src);
      const float zero = __shfl(my_zero[m], src);
      const float rstep = __shfl(my_rstep[m], src);
      const int h = kHalves == 2 ? (r8 >> 2) : 0;
      const float pw = float(1 << (BITS * (kHalves == 2 ? (r8 & 3) : r8)));
      const float lo = -zero, hi = qmax - zero;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q0 = wp[r8][i] * rstep;
        const float quo = __builtin_fmaf(__builtin_fmaf(-q0, step, wp[r8][i]), rstep, q0);
        const float cd = __builtin_amdgcn_fmed3f(__builtin_rintf(quo), lo, hi);
        acc[h][i] = __builtin_fmaf(cd, pw, acc[h][i]);
      }
      zacc[h] = __builtin_fmaf(zero, pw, zacc[h]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t wd = uint32_t(acc[0][i] + zacc[0]);
      if constexpr (kHalves == 2) wd |= uint32_t(acc[1][i] + zacc[1]) << 16;
      words[c * 8 + i][j] = wd;
    }
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
  dim3 grid(unsigned(K / kTile), unsigned((N + kRows - 1) / kRows));
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
