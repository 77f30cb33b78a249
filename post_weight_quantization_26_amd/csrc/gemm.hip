// Step 5 — the search GEMM: output error energy of every candidate.
//
//   partials[mt][c] = Σ_{t in token tile mt} ( Σ_k X[t][k] · E[c][k] )²
//
// E stacks the candidates' error weights [n_cand·N, K], so one launch covers
// the whole grid and every X tile is reused across all candidates ("05 —
// AWQ", section 4: for each α, scale, quantise and measure the output MSE;
// the product X·E_cᵀ is Y_c - Y). No output tile is ever written: the
// epilogue squares the fp32 accumulators and sums them per output column.
//
// bf16 path (gfx950 MFMA): 256x256 block tile, BK = 64, four wavefronts in a
// 2x2 arrangement, each owning a 128x128 sub-tile held as 4x4
// v_mfma_f32_32x32x16_bf16 accumulators (256 AGPRs). Both operands are
// K-contiguous, so one 16-byte LDS read per lane feeds an MFMA operand.
// Tiles are double-buffered in LDS with an XOR swizzle on 16-byte chunks
// (conflict-free ds_read_b128 for the 32 rows of a fragment). Workgroups are
// mapped so each XCD works on 4 token tiles x 8 candidate tiles at a time
// while all XCDs share the same 8 candidate tiles (one HBM read of each E
// panel per group of 32 token tiles, X panels reused from the last-level
// cache).
//
// fp32 path: a plain LDS-tiled FMA kernel (64x64 tiles), used for float32
// layers, where exact-ish float32 products are wanted and the work is small.
#include "device_common.h"

namespace awq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NT = 256;
constexpr int CHUNKS = BK / 8;  // 16-byte chunks per tile row

__device__ __forceinline__ int swz(int row, int chunk) { return row * CHUNKS + (chunk ^ (row & 7)); }

// Block id -> (token tile, candidate-column tile). Returns false for padding blocks.
__device__ __forceinline__ bool tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  if (tiles_m >= 32) {
    const int w = bid >> 8, j = bid & 255;
    const int xcd = j & 7, i = j >> 3;  // consecutive ids go round-robin over the 8 XCDs
    const int nwn = (tiles_n + 7) >> 3;
    const int g = w / nwn, wn = w - g * nwn;
    tm = 32 * g + 4 * xcd + (i & 3);
    tn = 8 * wn + (i >> 2);
  } else {
    tm = bid % tiles_m;
    tn = bid / tiles_m;
  }
  return tm < tiles_m && tn < tiles_n;
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void search_gemm_bf16_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ E,
                             int64_t M, int64_t Nc, int64_t K, int tiles_m, int tiles_n,
                             float* __restrict__ partials) {
  extern __shared__ uint4 smem[];
  // LDS: A buffers [2][BM*CHUNKS] then B buffers [2][BN*CHUNKS].
  uint4* const As0 = smem;
  uint4* const Bs0 = smem + 2 * BM * CHUNKS;

  int tm, tn;
  if (!tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Global -> register staging: thread loads chunk (tid & 7) of rows tid/8 + 32 i.
  const int ld_chunk = tid & 7;
  const int ld_row = tid >> 3;
  const uint4* gA[8];
  const uint4* gB[8];
  bool okA[8], okB[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t ra = m0 + ld_row + 32 * i, rb = n0 + ld_row + 32 * i;
    okA[i] = ra < M;
    okB[i] = rb < Nc;
    gA[i] = reinterpret_cast<const uint4*>(X + (okA[i] ? ra : 0) * K) + ld_chunk;
    gB[i] = reinterpret_cast<const uint4*>(E + (okB[i] ? rb : 0) * K) + ld_chunk;
  }
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  uint4 ra[8], rb[8];

  auto load_tile = [&](int64_t kt) {
    const int64_t off = kt * CHUNKS;  // in uint4 units
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ra[i] = okA[i] ? gA[i][off] : zero4;
      rb[i] = okB[i] ? gB[i][off] : zero4;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = ld_row + 32 * i;
      As0[buf * BM * CHUNKS + swz(row, ld_chunk)] = ra[i];
      Bs0[buf * BN * CHUNKS + swz(row, ld_chunk)] = rb[i];
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int64_t KT = K / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int frag_row = lane & 31;
  const int frag_half = lane >> 5;
  for (int64_t kt = 0; kt < KT; ++kt) {
    const int buf = int(kt & 1);
    if (kt + 1 < KT) load_tile(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ch = 2 * ks + frag_half;
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = __builtin_bit_cast(bf16x8_t,
                                  As0[buf * BM * CHUNKS + swz(wm * 128 + i * 32 + frag_row, ch)]);
        b[i] = __builtin_bit_cast(bf16x8_t,
                                  Bs0[buf * BN * CHUNKS + swz(wn * 128 + i * 32 + frag_row, ch)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: each lane's 16 accumulators of sub-tile (i, j) all lie in output
  // column j*32 + lane%32 of the wave's range; lanes l and l^32 share it.
  float* red = reinterpret_cast<float*>(smem);  // [2][BN]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[i][j][v] * acc[i][j][v];
    s += __shfl_xor(s, 32);
    if (lane < 32) red[wm * BN + wn * 128 + j * 32 + lane] = s;
  }
  __syncthreads();
  const int64_t c = n0 + tid;
  if (c < Nc) partials[int64_t(tm) * Nc + c] = red[tid] + red[BN + tid];
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
                              int64_t K, float* partials, hipStream_t st) {
  if (dtype == 1) {
    const int tiles_m = int((M + BM - 1) / BM), tiles_n = int((Nc + BN - 1) / BN);
    int64_t blocks;
    if (tiles_m >= 32)
      blocks = int64_t((tiles_m + 31) / 32) * 32 * (int64_t((tiles_n + 7) / 8) * 8);
    else
      blocks = int64_t(tiles_m) * tiles_n;
    const size_t lds = size_t(2) * (BM + BN) * CHUNKS * sizeof(uint4);  // 128 KiB
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(search_gemm_bf16_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    search_gemm_bf16_kernel<<<unsigned(blocks), NT, lds, st>>>(
        static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(E), M, Nc, K, tiles_m,
        tiles_n, partials);
  } else {
    const int64_t tiles_m = (M + FB - 1) / FB, tiles_n = (Nc + FB - 1) / FB;
    search_gemm_f32_kernel<<<unsigned(tiles_m * tiles_n), 256, 0, st>>>(
        static_cast<const float*>(X), static_cast<const float*>(E), M, Nc, K, tiles_m, partials);
  }
  return hipGetLastError();
}

}  // namespace awq
