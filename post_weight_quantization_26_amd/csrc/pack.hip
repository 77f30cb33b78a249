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
// A workgroup owns 128 output rows x one 128-channel tile of the input dim
// (1, 2 or 4 groups of g = 128, 64 or 32 channels): on the 70B-class layer
// 128-row tiles ran faster than 256-row ones (more resident waves per SIMD,
// a shorter tail of the grid). Lane (c, jb) takes 8 consecutive channels of
// one 8-row chunk; 16 lanes cover a row's 128 channels, so every load
// instruction reads whole 256-byte row segments. Loads are buffer loads
// (non-temporal: W is read once) from a per-workgroup base: one per-lane
// offset, the row step in the scalar offset, rows past N read as zero. All
// of a lane's loads are issued before any is used. Per 8-row chunk:
//   1. scaled weights w' = w·s of the 8 rows; each lane's partial range of
//      its 8 channels per row (max3/min3 chains, widened to contain 0);
//   2. the group ranges through LDS: every lane stores its 16 partials (8
//      row maxima, 8 negated row minima), lane c reads value c of all 16
//      lanes and reduces each group's kLanes of them; lanes c and c ^ 8
//      swap halves, so each lane holds (max, min) of row c % 8 in every
//      group;
//   3. each (row, group) pair's step and zero point (IEEE float32 divisions)
//      on one lane (lanes c and c ^ 8 split the groups; with one group they
//      duplicate), stored with the reciprocal split in two, 1/step ≈ rh + rl
//      (rl = fl32((1 - rh·step)·rh), the residual exact by FMA), and the code
//      bounds; every lane reads back the 8 rows of its group;
//   4. codes: quotient q = fma(w', rh, w'·rl), the float32 value of
//      w'·(rh + rl) = w'/step·(1 + O(2^-47)), so it is the correctly rounded
//      quotient unless the exact one lies within 2^-47 (relative) of a
//      float32 rounding midpoint; then it is the neighbouring float32, and
//      rint can differ from the oracle's only when that quotient is within
//      one ulp (< 1e-6 for codes below 16) of a .5 boundary. rint, clamp to
//      [-zero, qmax - zero], packed in exact float arithmetic (small
//      integers times powers of two, sums below 2^24): each word starts from
//      its rows' zero points Σ zero·base^row (read from LDS before the codes)
//      and takes acc = fma(code - zero, base^row, acc) row by row; 4-bit
//      words use two 16-bit halves.
// The partial words are transposed through LDS: for 4 bits each is one
// qweight word; for 3 bits four of them (32 rows) make three words. qweight
// rows are written with consecutive stores (4 bits: buffer stores from the
// tile's first row, the row step in the scalar offset).
#include "device_common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 128;   // input channels per workgroup

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Raw 16-byte pieces of 8 consecutive elements (one piece for 16-bit types,
// two for float32) and their conversion to float32.
template <int DT>
struct Raw8 {
  uint4 q[DT == 0 ? 2 : 1];
};

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 2 /* nt */);
  return make_uint4(t.x, t.y, t.z, t.w);
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

// Row parameters of one (row, group): reciprocal halves and code bounds.
struct alignas(16) RowPrm {
  float rh, rl, lo, hi;   // 1/step ≈ rh + rl; codes - zero in [lo, hi]
};

// The group ranges and row parameters are exchanged through LDS among the 16
// lanes of one chunk, which belong to one wavefront: a wavefront's LDS
// operations complete in issue order, so a fence that keeps the compiler
// from moving memory operations across it is all the exchange needs.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS slot of partial v (0..7 row maxima, 8..15 negated row minima) written
// by lane c of chunk jb: the 16 lanes' values of one v are 16 consecutive
// floats (one 64-byte read), and chunk slices are 272 floats apart so the
// four chunks of a wave write to different banks.
constexpr int kRedStride = 272;

template <int DT, int BITS, int G>
__global__ __launch_bounds__(kThreads) void pack_kernel(
    const void* __restrict__ W, int64_t N, int64_t K, const float* __restrict__ s,
    const float* __restrict__ ratio, int zero_point, int32_t* __restrict__ qweight,
    int32_t* __restrict__ qzeros, uint16_t* __restrict__ scales, int* __restrict__ overflow) {
#pragma clang fp contract(off)
  constexpr int kGroups = kTile / G;       // groups per tile
  constexpr int kLanes = G / 8;            // lanes per group
  constexpr int kHalves = BITS == 4 ? 2 : 1;
  constexpr int kRows = 128;               // output rows per workgroup
  constexpr int kChunks = 16;              // 8-row chunks per workgroup
  constexpr int kMine = kGroups >= 2 ? kGroups / 2 : 1;   // (row, group) pairs per lane
  constexpr int ESZ = DT == 0 ? 4 : 2;
  __shared__ uint32_t words[kTile][kChunks + 1];
  __shared__ uint16_t sc_lds[kGroups][kRows];
  __shared__ uint8_t z_lds[kGroups][kRows];
  __shared__ __attribute__((aligned(16))) float red[16 * kRedStride];
  __shared__ RowPrm prm[16][kGroups][8];
  __shared__ __attribute__((aligned(16))) float zlo[16][kGroups][8];   // -zero per row

  const int tid = threadIdx.x;
  const int c = tid & 15, jb = tid >> 4;
  const int gi = c / kLanes;                       // this lane's group within the tile
  const int64_t n0 = int64_t(blockIdx.y) * kRows;
  const int64_t tile = blockIdx.x;
  const int64_t k = tile * kTile + c * 8;

  float sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = s[k + i];

  // W rows n0 .. n0 + kRows - 1 from this workgroup's base; rows past N read
  // as zero. Offsets stay below 2^31 (the host checks 512·K < 2^31).
  const int64_t rows_here = N - n0 < kRows ? N - n0 : kRows;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(W) + n0 * K * ESZ), 0,
      int(rows_here * K * ESZ), 0x00020000);
  const int row_bytes = int(K) * ESZ;
  const int voff = (8 * jb * row_bytes) + int(k) * ESZ;

  // Every load is issued before any is used.
  Raw8<DT> raw[8];
#pragma unroll
  for (int r8 = 0; r8 < 8; ++r8) {
    const int soff = r8 * row_bytes;               // uniform: the scalar offset
#pragma unroll
    for (int q = 0; q < (DT == 0 ? 2 : 1); ++q)
      raw[r8].q[q] = buf_load16(rs, voff + 16 * q, soff);
  }

  const float qmax = float((1 << BITS) - 1);
  {
    const int j = jb;                              // this lane's 8-row chunk
    // 1. scaled weights and this lane's partial ranges
    float wp[8][8], mx[8], nmn[8];
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      float w[8];
      raw_to_f32<DT>(raw[r8], w);
#pragma unroll
      for (int i = 0; i < 8; ++i) wp[r8][i] = w[i] * sv[i];
      float a = fmaxf(fmaxf(0.f, wp[r8][0]), wp[r8][1]);
      float b = fminf(fminf(0.f, wp[r8][0]), wp[r8][1]);
#pragma unroll
      for (int i = 2; i < 8; i += 2) {
        a = fmaxf(fmaxf(a, wp[r8][i]), wp[r8][i + 1]);
        b = fminf(fminf(b, wp[r8][i]), wp[r8][i + 1]);
      }
      mx[r8] = a;
      nmn[r8] = -b;
    }
    // 2. group ranges through LDS
    float* my = red + jb * kRedStride + c;
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      my[16 * r8] = mx[r8];
      my[16 * (8 + r8)] = nmn[r8];
    }
    wave_lds_sync();
    // lane c reduces value c of the 16 lanes, kLanes at a time (one group
    // per run of kLanes lanes)
    float gm[kGroups];
    {
      const float4* rd = reinterpret_cast<const float4*>(red + jb * kRedStride + 16 * c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 t = rd[q];
        const int g = 4 * q / kLanes;
        const float m4 = fmaxf(fmaxf(t.x, t.y), fmaxf(t.z, t.w));
        if constexpr (kLanes == 4) {
          gm[g] = m4;
        } else {
          gm[g] = (4 * q) % kLanes == 0 ? m4 : fmaxf(gm[g], m4);
        }
      }
    }
    float gmx[kGroups], gmn[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const float m = gm[g];
      // lanes c and c ^ 8 hold the max and the negated min of row c % 8
      const float o = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
          __builtin_bit_cast(int, m), 0x128 /* row_ror:8 */, 0xF, 0xF, true));
      gmx[g] = c < 8 ? m : o;
      gmn[g] = -(c < 8 ? o : m);
    }
    // 3. the step, zero point and reciprocal halves of this lane's pairs
    const int r8 = c & 7;
    const int64_t n = n0 + 8 * j + r8;
    const bool valid = n < N;
    const float rr = (ratio != nullptr && valid) ? ratio[n] : 1.f;
#pragma unroll
    for (int m = 0; m < kMine; ++m) {
      const int g = kGroups >= 2 ? (c >> 3) + 2 * m : 0;
      const QParams p = group_qparams(gmx[g], gmn[g], rr, BITS, zero_point);
      const float rh = 1.0f / p.step;
      const float rl = __builtin_fmaf(-rh, p.step, 1.0f) * rh;
      if (kGroups >= 2 || c < 8) {
        prm[jb][g][r8] = RowPrm{rh, rl, -p.zero, qmax - p.zero};
        zlo[jb][g][r8] = -p.zero;
        const uint16_t hb = __builtin_bit_cast(uint16_t, _Float16(p.step));
        sc_lds[g][8 * j + r8] = hb;
        z_lds[g][8 * j + r8] = uint8_t(p.zero);
        if (valid && (hb & 0x7FFFu) >= 0x7C00u) *overflow = 1;
      }
    }
    wave_lds_sync();
    // 4. codes of the 8 rows, packed exactly in float. Each word (half
    //    word for 4 bits) starts from its rows' zero points, zacc =
    //    Σ_r zero_r·base^r, and adds (code_r - zero_r)·base^r row by row:
    //    every partial sum is an integer in [0, 2^24), so the order of the
    //    additions does not change the result.
    float zacc[kHalves];
    {
      const float4* zl = reinterpret_cast<const float4*>(&zlo[jb][gi][0]);
      const float4 za = zl[0], zb = zl[1];
      const float nz[8] = {za.x, za.y, za.z, za.w, zb.x, zb.y, zb.z, zb.w};
#pragma unroll
      for (int h = 0; h < kHalves; ++h) zacc[h] = 0.f;
#pragma unroll
      for (int q8 = 0; q8 < 8; ++q8) {
        const int h = kHalves == 2 ? (q8 >> 2) : 0;
        const float pw = float(1 << (BITS * (kHalves == 2 ? (q8 & 3) : q8)));
        zacc[h] = __builtin_fmaf(-nz[q8], pw, zacc[h]);
      }
    }
    float acc[kHalves][8];
#pragma unroll
    for (int q8 = 0; q8 < 8; ++q8) {
      const RowPrm pr = prm[jb][gi][q8];
      const int h = kHalves == 2 ? (q8 >> 2) : 0;
      const int r = kHalves == 2 ? (q8 & 3) : q8;
      const float pw = float(1 << (BITS * r));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float quo = __builtin_fmaf(wp[q8][i], pr.rh, wp[q8][i] * pr.rl);
        const float cd = __builtin_amdgcn_fmed3f(__builtin_rintf(quo), pr.lo, pr.hi);
        acc[h][i] = r == 0 ? cd + zacc[h] : __builtin_fmaf(cd, pw, acc[h][i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t wd = uint32_t(acc[0][i]);
      if constexpr (kHalves == 2) wd |= uint32_t(acc[1][i]) << 16;
      words[c * 8 + i][j] = wd;
    }
  }
  __syncthreads();

  const int64_t g0 = tile * kGroups;               // first group row of this tile
  if constexpr (BITS == 4) {
    const int64_t N8 = N / 8;
    const int jj = tid % kChunks;
    const int64_t jcol = n0 / 8 + jj;
    if (jcol < N8) {
      // from this tile's first qweight row; row steps go in the scalar
      // offset (the host checks that 4·K·N/8 stays below 2^31 bytes)
      const __amdgpu_buffer_rsrc_t qs = __builtin_amdgcn_make_buffer_rsrc(
          qweight + tile * kTile * N8, 0, int(kTile * N8 * 4), 0x00020000);
      const int kk0 = tid / kChunks;
      const int qoff = int((kk0 * N8 + jcol) * 4);
#pragma unroll
      for (int v = 0; v < kChunks / 2; ++v) {
        const int kk = kk0 + (kThreads / kChunks) * v;
        __builtin_amdgcn_raw_buffer_store_b32(words[kk][jj], qs, qoff,
                                              int((kThreads / kChunks) * v * N8 * 4), 0);
      }
    }
    const int zg = tid / kChunks;
    if (zg < kGroups && jcol < N8) {
      uint32_t zw = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) zw |= uint32_t(z_lds[zg][8 * jj + i]) << (4 * i);
      qzeros[(g0 + zg) * N8 + jcol] = int32_t(zw);
    }
  } else {
    // 3 bits: four 24-bit partial words (rows 32q .. 32q+31) -> three words.
    constexpr int kQ = kChunks / 4;              // 32-row column blocks per workgroup
    const int64_t N32 = N / 32, N3 = N32 * 3;
    const int q = tid % kQ;
    const int64_t qcol = n0 / 32 + q;
    if (qcol < N32) {
#pragma unroll
      for (int v = 0; v < kTile * kQ / kThreads; ++v) {
        const int kk = tid / kQ + (kThreads / kQ) * v;
        const uint32_t a = words[kk][4 * q], b = words[kk][4 * q + 1];
        const uint32_t cc = words[kk][4 * q + 2], d = words[kk][4 * q + 3];
        int32_t* dst = qweight + (tile * kTile + kk) * N3 + 3 * qcol;
        dst[0] = int32_t(a | (b << 24));
        dst[1] = int32_t((b >> 8) | (cc << 16));
        dst[2] = int32_t((cc >> 16) | (d << 8));
      }
    }
    const int zg = tid / kQ;
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
  if (tid < kRows) {
#pragma unroll
    for (int zg = 0; zg < kGroups; ++zg)
      if (n0 + tid < N) scales[(g0 + zg) * N + n0 + tid] = sc_lds[zg][tid];
  }
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
  dim3 grid(unsigned(K / kTile), unsigned((N + 127) / 128));
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
