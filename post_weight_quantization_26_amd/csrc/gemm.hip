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
// the A operand and E as B, in a persistent grid of one workgroup per CU
// whose tiles follow one another through the ring.
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

// The epilogue's column sums of the two wave rows (not aliased with the
// k-tile ring, which already holds the next tile's first k-tile).
__shared__ float sRed[2 * BN];

// Operand contexts of output tile (tm, tn).
template <bool SPLIT>
__device__ __forceinline__ void search_tile_setup(GemmCtx64& c, const uint16_t* X,
                                                  const uint16_t* E, int64_t M, int64_t Nc,
                                                  int64_t K, int tm, int tn) {
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;
  const int64_t rows_a = M - m0 < BM ? M - m0 : BM;
  const int64_t rows_b = Nc - n0 < BN ? Nc - n0 : BN;
  if (SPLIT)
    gemm_setup64(c, X + m0 * K, rows_a, K, E + n0 * 2 * K, rows_b, 2 * K, 2 * K, false, true);
  else
    gemm_setup64(c, X + m0 * K, rows_a, E + n0 * K, rows_b, K);
}

// First block id at or after bid, in steps of the grid size, that maps to a
// tile; nblocks if none.
__device__ __forceinline__ int64_t next_tile(int64_t bid, int64_t nblocks, int tiles_m,
                                             int tiles_n, int& tm, int& tn) {
  for (; bid < nblocks; bid += gridDim.x)
    if (tile_of(int(bid), tiles_m, tiles_n, tm, tn)) break;
  return bid;
}

// K must be a multiple of 128 (the entry points check it), so every tile's
// k-loop has an even number of 64-wide k-tiles. F16: fp16 operands instead
// of bf16 (the same tile, the fp16 MFMA). SPLIT: E rows are hi/lo halves of
// length 2K.
//
// Persistent: workgroup b takes block ids b, b + grid, b + 2·grid, ... of the
// tile_of order (with a grid of 256 that keeps each block id's XCD). Each
// tile's last k-tile region copies the first k-tile of the workgroup's next
// tile, so only the first tile waits for its operands.
template <bool F16, bool SPLIT>
__device__ __forceinline__ void search_gemm_16(const uint16_t* __restrict__ X,
                                               const uint16_t* __restrict__ E, int64_t M,
                                               int64_t Nc, int64_t K, int tiles_m, int tiles_n,
                                               int64_t nblocks, float* __restrict__ partials) {
  int tm = 0, tn = 0;
  int64_t bid = next_tile(blockIdx.x, nblocks, tiles_m, tiles_n, tm, tn);
  if (bid >= nblocks) return;
  GemmCtx64 c;
  search_tile_setup<SPLIT>(c, X, E, M, Nc, K, tm, tn);
  dma64<0>(c, 0);
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  region_barrier();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wm = c.wave >> 1, wn = c.wave & 1;
  for (;;) {
    int ntm = tm, ntn = tn;
    const int64_t nbid = next_tile(bid + gridDim.x, nblocks, tiles_m, tiles_n, ntm, ntn);
    const bool more = nbid < nblocks;
    // after the last tile the copies re-read this tile's first k-tile (unused)
    GemmCtx64 cn = c;
    if (more) search_tile_setup<SPLIT>(cn, X, E, M, Nc, K, ntm, ntn);
    floatx4 acc[8][8];
    gemm_mainloop16_chain<F16>(c, cn, acc);
    column_square_sums(acc, sRed, wm, wn, lane);
    __syncthreads();
    const int64_t col = int64_t(tn) * BN + tid;
    if (col < Nc) partials[int64_t(tm) * Nc + col] = sRed[tid] + sRed[BN + tid];
    if (!more) break;
    bid = nbid;
    tm = ntm;
    tn = ntn;
    c = cn;
  }
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void search_gemm_bf16_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ E,
                             int64_t M, int64_t Nc, int64_t K, int tiles_m, int tiles_n,
                             int64_t nblocks, float* __restrict__ partials) {
  search_gemm_16<false, false>(X, E, M, Nc, K, tiles_m, tiles_n, nblocks, partials);
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void search_gemm_f16_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ E,
                            int64_t M, int64_t Nc, int64_t K, int tiles_m, int tiles_n,
                            int64_t nblocks, float* __restrict__ partials) {
  search_gemm_16<true, false>(X, E, M, Nc, K, tiles_m, tiles_n, nblocks, partials);
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void search_gemm_bf16_split_kernel(const uint16_t* __restrict__ X,
                                   const uint16_t* __restrict__ E, int64_t M, int64_t Nc,
                                   int64_t K, int tiles_m, int tiles_n, int64_t nblocks,
                                   float* __restrict__ partials) {
  search_gemm_16<false, true>(X, E, M, Nc, K, tiles_m, tiles_n, nblocks, partials);
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void search_gemm_f16_split_kernel(const uint16_t* __restrict__ X,
                                  const uint16_t* __restrict__ E, int64_t M, int64_t Nc,
                                  int64_t K, int tiles_m, int tiles_n, int64_t nblocks,
                                  float* __restrict__ partials) {
  search_gemm_16<true, true>(X, E, M, Nc, K, tiles_m, tiles_n, nblocks, partials);
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

// Workgroups of the persistent search GEMM: 256, a multiple of the 8 XCDs,
// so workgroup b runs on the XCD that block ids b + 256·i are mapped for.
constexpr int64_t kSearchGrid = 256;

hipError_t launch_search_gemm(const void* X, int dtype, const void* E, int64_t M, int64_t Nc,
                              int64_t K, int split, float* partials, hipStream_t st) {
  if (dtype == 1 || dtype == 2) {
    if (K % 128) return hipErrorInvalidValue;
    const int tiles_m = int((M + BM - 1) / BM), tiles_n = int((Nc + BN - 1) / BN);
    const int64_t blocks = gemm_blocks(tiles_m, tiles_n);
    // one workgroup per CU of a 256-CU part, each looping over its tiles
    const unsigned grid = unsigned(blocks < kSearchGrid ? blocks : kSearchGrid);
    const uint16_t* x = static_cast<const uint16_t*>(X);
    const uint16_t* e = static_cast<const uint16_t*>(E);
    if (dtype == 1 && split)
      search_gemm_bf16_split_kernel<<<grid, NT, 0, st>>>(x, e, M, Nc, K, tiles_m, tiles_n, blocks,
                                                         partials);
    else if (dtype == 1)
      search_gemm_bf16_kernel<<<grid, NT, 0, st>>>(x, e, M, Nc, K, tiles_m, tiles_n, blocks,
                                                   partials);
    else if (split)
      search_gemm_f16_split_kernel<<<grid, NT, 0, st>>>(x, e, M, Nc, K, tiles_m, tiles_n, blocks,
                                                        partials);
    else
      search_gemm_f16_kernel<<<grid, NT, 0, st>>>(x, e, M, Nc, K, tiles_m, tiles_n, blocks,
                                                  partials);
  } else {
    const int64_t tiles_m = (M + FB - 1) / FB, tiles_n = (Nc + FB - 1) / FB;
    search_gemm_f32_kernel<<<unsigned(tiles_m * tiles_n), 256, 0, st>>>(
        static_cast<const float*>(X), static_cast<const float*>(E), M, Nc, K, tiles_m, partials);
  }
  return hipGetLastError();
}

}  // namespace awq
