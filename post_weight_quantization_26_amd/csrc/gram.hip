// The search's output errors through the Gram matrix of the activations:
//
//   M_n = Σ_t (Σ_k X[t][k]·E[n][k])² = E_n · G · E_nᵀ,   G = XᵀX  [K, K]
//
// (an exact identity of the error the pages measure: "05 — AWQ: Activation-
// Aware Weight Scaling", section 4, quantise and measure the output MSE).
// G costs 2·T·K² once per layer; each candidate row then costs 2·K² instead
// of 2·T·K, T/K times less (16x at 64K tokens and K = 4096).
//
//  1. transpose_pad_kernel: Xt [K, Tp] = Xᵀ with the token dim padded to a
//     multiple of 128 with zeros (zero rows do not change G).
//  2. gram_partial_kernel: G is symmetric, so only its 256x256 tiles on and
//     above the diagonal are formed, on the shared MFMA main loop
//     (gemm_core.h). To keep every CU busy the token range is split into S
//     slices (S chosen on the host to balance whole rounds of work); each
//     (tile, slice) unit stores its float32 partial tile.
//     gram_reduce_kernel adds a tile's S partials in a fixed order and stores
//     it as two bf16 halves, hi = bf16(G) and lo = bf16(G - hi) (hi + lo
//     carries G to about 2^-16 relative, so the bf16 MFMA that follows does
//     not lose G's precision). Tiles above the diagonal are stored doubled
//     (exact), and only the upper tiles are stored at all, because
//       e·G·eᵀ = Σ_tm [ e_tm·G_tm,tm·e_tmᵀ + Σ_{tn > tm} e_tm·(2·G_tm,tn)·e_tnᵀ ]
//     over the 256-wide index tiles. Row j of Gs [K, 2K + 256] holds, for each
//     128-wide block c of columns, hi then lo of that block:
//       Gs[j][256·c + w] = hi(G'[j][128·c + w]), Gs[j][256·c + 128 + w] = lo(...)
//     so row tile tm's part from its diagonal tile on is one contiguous run.
//  3. gram_search_kernel: for a batch of candidate error rows E [Nc, K]
//     (bf16, the same operands the direct search GEMM uses), row tile tm
//     runs one k-loop over Gs columns [512·tm, 2K) with each 128-wide block
//     of E (from column 256·tm) read twice, once against hi and once
//     against lo: Z[j][n] = Σ_{i >= 256·tm} G'[j][i]·E[n][i] in float32. The
//     epilogue multiplies each Z[j][n] by E[n][j] and sums over the tile's
//     rows j: partials[tm][n]; the row reduction over tiles gives M_n. The
//     k-loop of row tile tm is 2·(K - 256·tm) long, about half the full
//     product on average; row tiles tm and nt - 1 - tm share a workgroup so
//     that every workgroup does the same work.
#include "gemm_core.h"

namespace awq {
namespace {

// ---------------------------------------------------------------------------
// 1. Xt = Xᵀ, token dim padded with zeros
// ---------------------------------------------------------------------------

// Workgroup = 64 tokens x 64 channels through LDS; 16-byte loads and stores.
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ X,
                                                            int64_t T, int64_t K, int64_t Tp,
                                                            int64_t ldx,
                                                            uint16_t* __restrict__ Xt) {
  __shared__ uint16_t tile[64][72];
  const int64_t t0 = int64_t(blockIdx.x) * 64, k0 = int64_t(blockIdx.y) * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + 256 * u;         // 512 chunks of 8 channels
    const int r = e >> 3, c8 = (e & 7) * 8;
    const int64_t t = t0 + r;
    uint4 q = make_uint4(0, 0, 0, 0);
    if (t < T) q = *reinterpret_cast<const uint4*>(X + t * K + k0 + c8);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[r][c8 + 2 * i] = uint16_t(w[i] & 0xFFFFu);
      tile[r][c8 + 2 * i + 1] = uint16_t(w[i] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + 256 * u;         // 512 chunks of 8 tokens
    const int kr = e >> 3, t8 = (e & 7) * 8;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = uint32_t(tile[t8 + 2 * i][kr]) | (uint32_t(tile[t8 + 2 * i + 1][kr]) << 16);
    if (t0 + t8 < Tp)
      *reinterpret_cast<uint4*>(Xt + (k0 + kr) * ldx + t0 + t8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---------------------------------------------------------------------------
// 2. G = Xt·Xtᵀ: upper tiles x token slices, then the slice sum as hi/lo halves
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint16_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Upper tile u (row-major over tm <= tn of an nt x nt grid) -> (tm, tn).
__device__ __forceinline__ void upper_tile(int u, int nt, int& tm, int& tn) {
  int r = 0, first = 0;
  while (first + (nt - r) <= u) {
    first += nt - r;
    ++r;
  }
  tm = r;
  tn = r + (u - first);
}

// Block b: slice s = b / U, upper tile u = b % U (units of one token slice run
// together, so concurrent blocks share that slice's panels of Xt).
// P[(s·U + u)][256·256]: float32 partial tile, row-major.
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gram_partial_kernel(const uint16_t* __restrict__ Xt, int64_t K, int64_t ldx, int64_t Ts,
                         int nt, int U, float* __restrict__ P) {
  const int s = blockIdx.x / U, u = blockIdx.x % U;
  int tm, tn;
  upper_tile(u, nt, tm, tn);
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;
  const int64_t rows_a = K - m0 < BM ? K - m0 : BM;
  const int64_t rows_b = K - n0 < BN ? K - n0 : BN;
  const int64_t t0 = int64_t(s) * Ts;
  GemmCtx64 c;
  gemm_setup64(c, Xt + m0 * ldx + t0, rows_a, ldx, Xt + n0 * ldx + t0, rows_b, ldx, Ts, false);
  floatx4 acc[8][8];
  gemm_mainloop16<false>(c, acc);

  // lane l of block (i, j) holds column l % 16 and rows 4·(l/16) + v
  const int lane = threadIdx.x & 63;
  const int wm = c.wave >> 1, wn = c.wave & 1;
  float* tile = P + (int64_t(s) * U + u) * (BM * BN);
  const int row0 = wm * 128 + 4 * (lane >> 4);
  const int col0 = wn * 128 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        tile[(row0 + i * 16 + v) * BN + col0 + j * 16] = acc[i][j][v];
}

// Block (u, sb): the 64x64 sub-block sb of upper tile u. Thread t takes row
// t / 4 and 16 consecutive columns; the S partials are added in slice order.
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float* __restrict__ P, int S,
                                                          int U, int nt, int64_t K, int64_t ldg,
                                                          uint16_t* __restrict__ Gs) {
#pragma clang fp contract(off)
  const int u = blockIdx.x, sb = blockIdx.y;
  int tm, tn;
  upper_tile(u, nt, tm, tn);
  const int sr = (sb >> 2) * 64, sc = (sb & 3) * 64;
  const int t = threadIdx.x, r = t >> 2, c0 = (t & 3) * 16;
  float g[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) g[e] = 0.f;
  for (int sl = 0; sl < S; ++sl) {
    const float4* src = reinterpret_cast<const float4*>(
        P + (int64_t(sl) * U + u) * (BM * BN) + (sr + r) * BN + sc + c0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = src[q];
      g[4 * q] += v.x; g[4 * q + 1] += v.y; g[4 * q + 2] += v.z; g[4 * q + 3] += v.w;
    }
  }
  uint16_t hi[16], lo[16];
  const float w = tm < tn ? 2.f : 1.f;   // tiles above the diagonal count twice (exact)
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float f = g[e] * w;
    hi[e] = bf16_bits(f);
    lo[e] = bf16_bits(f - __uint_as_float(uint32_t(hi[e]) << 16));
  }
  const int64_t R = int64_t(tm) * BM + sr + r, C = int64_t(tn) * BN + sc + c0;
  if (R < K && C < K) {   // K is a multiple of 128, so 16 columns are all in or all out
    uint32_t wh[8], wl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      wh[e] = uint32_t(hi[2 * e]) | (uint32_t(hi[2 * e + 1]) << 16);
      wl[e] = uint32_t(lo[2 * e]) | (uint32_t(lo[2 * e + 1]) << 16);
    }
    // the 16 columns lie in one 128-wide block (c0 is a multiple of 16)
    const int64_t col = (C >> 7) * 256 + (C & 127);
    uint4* dh = reinterpret_cast<uint4*>(Gs + R * ldg + col);
    uint4* dl = reinterpret_cast<uint4*>(Gs + R * ldg + col + 128);
    dh[0] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
    dh[1] = make_uint4(wh[4], wh[5], wh[6], wh[7]);
    dl[0] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
    dl[1] = make_uint4(wl[4], wl[5], wl[6], wl[7]);
  }
}

// ---------------------------------------------------------------------------
// 3. candidates: partials[tm][n] = Σ_{j in row tile tm} Z[j][n] · E[n][j]
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gram_search_kernel(const uint16_t* __restrict__ Gs, int64_t ldg, const uint16_t* __restrict__ E,
                        int64_t K, int64_t Nc, int tiles_m, int tiles_n,
                        float* __restrict__ partials) {
  // Row tiles p and tiles_m - 1 - p run in one workgroup, one after the
  // other: their k-loops add up to (tiles_m + 1)·256 columns of K for every
  // p, so all workgroups take about the same time. Groups of 8 candidate
  // tiles; consecutive blocks go round-robin over the 8 XCDs, so each XCD
  // keeps one E tile for all row tiles of a group.
  const int pairs = (tiles_m + 1) >> 1;
  const int per = 8 * pairs;
  const int g = int(blockIdx.x) / per, rem = int(blockIdx.x) - g * per;
  const int p = rem >> 3, tn = 8 * g + (rem & 7);
  if (tn >= tiles_n) return;
  const int n_half = (tiles_m - 1 - p == p) ? 1 : 2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t n0 = int64_t(tn) * BN;
  const int64_t rows_b = Nc - n0 < BN ? Nc - n0 : BN;
  float* red = reinterpret_cast<float*>(s64A0);  // [2][BN]
#pragma nounroll
  for (int h = 0; h < n_half; ++h) {
    const int tm = h ? tiles_m - 1 - p : p;
    const int64_t m0 = int64_t(tm) * BM;
    const int64_t rows_a = K - m0 < BM ? K - m0 : BM;
    GemmCtx64 c;
    gemm_setup64(c, Gs + m0 * ldg + 2 * m0, rows_a, ldg, E + n0 * K + m0, rows_b, K,
                 2 * (K - m0), true);
    floatx4 acc[8][8];
    gemm_mainloop16<false>(c, acc);

    // Epilogue: lane l of block (i, j) holds column n = ... + l % 16 and
    // the 4 consecutive rows 4·(l/16) + v of the wave's 16-row block i,
    // which take one 8-byte load of E[n][rows].
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int wm = c.wave >> 1, wn = c.wave & 1;
    const int64_t row0 = m0 + wm * 128 + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = n0 + wn * 128 + j * 16 + (lane & 15);
      float s = 0.f;
      if (n < Nc) {
        const uint16_t* en = E + n * K;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int64_t r = row0 + i * 16;      // 4 consecutive rows r..r+3
          if (r < K) {
            const uint2 ev = *reinterpret_cast<const uint2*>(en + r);
            s += acc[i][j][0] * __uint_as_float(ev.x << 16);
            s += acc[i][j][1] * __uint_as_float(ev.x & 0xFFFF0000u);
            s += acc[i][j][2] * __uint_as_float(ev.y << 16);
            s += acc[i][j][3] * __uint_as_float(ev.y & 0xFFFF0000u);
          }
        }
      }
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (lane < 16) red[wm * BN + wn * 128 + j * 16 + lane] = s;
    }
    __syncthreads();
    const int64_t col = n0 + tid;
    if (col < Nc) partials[int64_t(tm) * Nc + col] = red[tid] + red[BN + tid];
    __syncthreads();  // red lives in LDS stage 0, which the next k-loop refills
  }
}

}  // namespace

// S token slices of Tp / S tokens each (Tp / S a multiple of 128); P holds
// S x (upper tiles) float32 partial tiles of 256 x 256.
hipError_t launch_gram_build(const void* X, int64_t T, int64_t K, int64_t Tp, int64_t ldx, int S,
                             uint16_t* Xt, float* P, int64_t ldg, uint16_t* Gs, hipStream_t st) {
  if (K % 128 || Tp % 128 || Tp < T || S < 1 || Tp % (int64_t(S) * 128) || ldx < Tp ||
      ldx % 8 || ldg < 2 * K || ldg % 8)
    return hipErrorInvalidValue;
  dim3 tgrid(unsigned((Tp + 63) / 64), unsigned(K / 64));
  transpose_pad_kernel<<<tgrid, 256, 0, st>>>(static_cast<const uint16_t*>(X), T, K, Tp, ldx, Xt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nt = int((K + BM - 1) / BM);
  const int U = nt * (nt + 1) / 2;
  gram_partial_kernel<<<unsigned(int64_t(U) * S), NT, 0, st>>>(Xt, K, ldx, Tp / S, nt, U, P);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  gram_reduce_kernel<<<dim3(unsigned(U), 16), 256, 0, st>>>(P, S, U, nt, K, ldg, Gs);
  return hipGetLastError();
}

hipError_t launch_gram_search(const uint16_t* Gs, int64_t ldg, const void* E, int64_t K, int64_t Nc,
                              float* partials, hipStream_t st) {
  if (K % 128) return hipErrorInvalidValue;
  const int tiles_m = int((K + BM - 1) / BM), tiles_n = int((Nc + BN - 1) / BN);
  const int64_t blocks = int64_t((tiles_m + 1) / 2) * 8 * ((tiles_n + 7) / 8);
  gram_search_kernel<<<unsigned(blocks), NT, 0, st>>>(
      Gs, ldg, static_cast<const uint16_t*>(E), K, Nc, tiles_m, tiles_n, partials);
  return hipGetLastError();
}

}  // namespace awq
