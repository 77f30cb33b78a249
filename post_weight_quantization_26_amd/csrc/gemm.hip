// Step 5 — the search GEMM: output error energy of every candidate.
//
//   partials[mt][c] = Σ_{t in token tile mt} ( Σ_k X[t][k] · E[c][k] )²
//
// E stacks the candidates' error weights [n_cand·N, K], so one launch covers
// the whole grid and every X tile is reused across all candidates ("05 —
// AWQ: Activation-Aware Weight Scaling", section 4: for each α, scale,
// quantise and measure the output MSE; the product X·E_cᵀ is Y_c - Y). No
// output tile is ever written: the epilogue squares the fp32 accumulators and
// sums them per output column.
//
// bf16 path: the 16x16x32 MFMA main loop of gemm_core.h (256x256 tiles,
// 2-stage LDS-DMA ring of 64-wide k-tiles, XCD-aware tile order) with X as
// the A operand and E as B.
// Each XCD runs 4 token tiles x 8 candidate tiles at a time while all XCDs
// share the same 8 candidate tiles (one E panel fetch per group of 32 token
// tiles; X panels stay in the last-level cache).
//
// Split operands: E may instead hold each candidate row as two 16-bit halves,
// hi = rnd(e) and lo = rnd(e - hi), alternating in 128-wide blocks
// [hi_0 | lo_0 | hi_1 | lo_1 | ...] (row length 2K). The main loop then reads
// each 128-wide block of X twice (its pair_a mode), so the accumulators hold
// X·(hi + lo)ᵀ: the candidate operand carries ~16 significand bits instead of
// 8 (bf16) or 11 (fp16), for twice the MFMA work.
//
// fp32 path: a plain LDS-tiled FMA kernel (64x64 tiles) for float32 layers.
#include "gemm_core.h"

namespace awq {
namespace {

// K must be a multiple of 128 (the entry points check it). F16: fp16
// operands instead of bf16 (the same tile, the fp16 MFMA). SPLIT: E rows are
// hi/lo halves of length 2K.
template <bool F16, bool SPLIT>
__device__ __forceinline__ void search_gemm_16(const uint16_t* __restrict__ X,
                                               const uint16_t* __restrict__ E, int64_t M,
                                               int64_t Nc, int64_t K, int tiles_m, int tiles_n,
                                               float* __restrict__ partials) {
  int tm, tn;
  if (!tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;
  const int64_t rows_a = M - m0 < BM ? M - m0 : BM;
  const int64_t rows_b = Nc - n0 < BN ? Nc - n0 : BN;
  GemmCtx64 c;
  if (SPLIT)
    gemm_setup64(c, X + m0 * K, rows_a, K, E + n0 * 2 * K, rows_b, 2 * K, 2 * K, false, true);
  else
    gemm_setup64(c, X + m0 * K, rows_a, E + n0 * K, rows_b, K);
  floatx4 acc[8][8];
  gemm_mainloop16<F16>(c, acc);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wm = c.wave >> 1, wn = c.wave & 1;

  // Epilogue: each lane's 4 accumulators of block (i, j) all lie in output
  // column j*16 + lane%16 of the wave's range; lanes l, l^16, l^32, l^48
  // share it.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float* red = reinterpret_cast<float*>(s64A0);  // [2][BN]
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) s += acc[i][j][v] * acc[i][j][v];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (lane < 16) red[wm * BN + wn * 128 + j * 16 + lane] = s;
  }
  __syncthreads();
  const int64_t col = n0 + tid;
  if (col < Nc) partials[int64_t(tm) * Nc + col] = red[tid] + red[BN + tid];
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void search_gemm_bf16_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ E,
                             int64_t M, int64_t Nc, int64_t K, int tiles_m, int tiles_n,
                             float* __restrict__ partials) {
  search_gemm_16<false, false>(X, E, M, Nc, K, tiles_m, tiles_n, partials);
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void search_gemm_f16_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ E,
                            int64_t M, int64_t Nc, int64_t K, int tiles_m, int tiles_n,
                            float* __restrict__ partials) {
  search_gemm_16<true, false>(X, E, M, Nc, K, tiles_m, tiles_n, partials);
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void search_gemm_bf16_split_kernel(const uint16_t* __restrict__ X,
                                   const uint16_t* __restrict__ E, int64_t M, int64_t Nc,
                                   int64_t K, int tiles_m, int tiles_n,
                                   float* __restrict__ partials) {
  search_gemm_16<false, true>(X, E, M, Nc, K, tiles_m, tiles_n, partials);
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void search_gemm_f16_split_kernel(const uint16_t* __restrict__ X,
                                  const uint16_t* __restrict__ E, int64_t M, int64_t Nc,
                                  int64_t K, int tiles_m, int tiles_n,
                                  float* __restrict__ partials) {
  search_gemm_16<true, true>(X, E, M, Nc, K, tiles_m, tiles_n, partials);
}

// ---------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------
constexpr int FB = 64;
constexpr int FK = 16;

__global__ __launch_bounds__(256) void search_gemm_f32_kernel(const float* __restrict__ X,
                                                              const float* __restrict__ E,
                                                              int64_t M, int64_t Nc, int64_t K,
                                                              int64_t tiles_m,
                                                              float* __restrict__ partials) {
  __shared__ float As[FK][FB + 4];
  __shared__ float Bs[FK][FB + 4];
  __shared__ float red[16][FB];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t bm = int64_t(blockIdx.x) % tiles_m, bn = int64_t(blockIdx.x) / tiles_m;
  const int64_t m0 = bm * FB, n0 = bn * FB;
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const bool okA = m0 + lr < M, okB = n0 + lr < Nc;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += FK) {
    const float4 a = okA ? *reinterpret_cast<const float4*>(X + (m0 + lr) * K + k0 + lk)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 b = okB ? *reinterpret_cast<const float4*>(E + (n0 + lr) * K + k0 + lk)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    As[lk + 0][lr] = a.x; As[lk + 1][lr] = a.y; As[lk + 2][lr] = a.z; As[lk + 3][lr] = a.w;
    Bs[lk + 0][lr] = b.x; Bs[lk + 1][lr] = b.y; Bs[lk + 2][lr] = b.z; Bs[lk + 3][lr] = b.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[kk][ty * 4 + i];
        bv[i] = Bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s += acc[i][j] * acc[i][j];
    red[ty][tx * 4 + j] = s;
  }
  __syncthreads();
  if (tid < FB) {
    float s = 0.f;
    for (int r = 0; r < 16; ++r) s += red[r][tid];
    if (n0 + tid < Nc) partials[bm * Nc + n0 + tid] = s;
  }
}

}  // namespace

hipError_t launch_search_gemm(const void* X, int dtype, const void* E, int64_t M, int64_t Nc,
                              int64_t K, int split, float* partials, hipStream_t st) {
  if (dtype == 1 || dtype == 2) {
    if (K % 128) return hipErrorInvalidValue;
    const int tiles_m = int((M + BM - 1) / BM), tiles_n = int((Nc + BN - 1) / BN);
    const int64_t blocks = gemm_blocks(tiles_m, tiles_n);
    const uint16_t* x = static_cast<const uint16_t*>(X);
    const uint16_t* e = static_cast<const uint16_t*>(E);
    if (dtype == 1 && split)
      search_gemm_bf16_split_kernel<<<unsigned(blocks), NT, 0, st>>>(x, e, M, Nc, K, tiles_m,
                                                                       tiles_n, partials);
    else if (dtype == 1)
      search_gemm_bf16_kernel<<<unsigned(blocks), NT, 0, st>>>(x, e, M, Nc, K, tiles_m, tiles_n,
                                                                 partials);
    else if (split)
      search_gemm_f16_split_kernel<<<unsigned(blocks), NT, 0, st>>>(x, e, M, Nc, K, tiles_m,
                                                                      tiles_n, partials);
    else
      search_gemm_f16_kernel<<<unsigned(blocks), NT, 0, st>>>(x, e, M, Nc, K, tiles_m, tiles_n,
                                                                partials);
  } else {
    const int64_t tiles_m = (M + FB - 1) / FB, tiles_n = (Nc + FB - 1) / FB;
    search_gemm_f32_kernel<<<unsigned(tiles_m * tiles_n), 256, 0, st>>>(
        static_cast<const float*>(X), static_cast<const float*>(E), M, Nc, K, tiles_m, partials);
  }
  return hipGetLastError();
}

}  // namespace awq
