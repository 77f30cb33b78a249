// Steps 4-5 in one kernel: the search GEMM with the candidates' error
// weights formed while the operand is staged ("05 — AWQ: Activation-Aware
// Weight Scaling", section 4: scale, quantise and measure the output error
// for every α; section 3 "The scaling trick" for the fold), instead of
// written to HBM by a separate transform pass first.
//
//   partials[mt][c·N + n] = Σ_{t in token tile mt} ( Σ_k X[t][k] · E_c[n][k] )²
//   E_c[n][k] = (q − zero)·step / s_c[k] − W[n][k],
//   q = clamp(rint(W[n][k]·s_c[k] / step) + zero, 0, 2^b − 1)
//
// with (step, zero, 1/step) of every (candidate, row, group) from the
// parameter pass (launch_group_params) and the arithmetic of the transform
// kernel, operation for operation, so the operand and the sums equal the
// two-pass path's bit for bit.
//
// The 256x256 tiles and 16x16x32 main loop of gemm_core.h: X's k-tiles come
// through the LDS-DMA ring; the B tile (256 rows of one candidate, N a
// multiple of 256) is formed in registers. Lane (j, kc) = (tid / 8, tid % 8)
// forms rows 8j .. 8j + 7 and k 8kc .. 8kc + 7 of each 64-wide k-tile: the 8
// lanes of an LDS write group store one row's 8 chunks (distinct banks), and
// read 128 consecutive bytes of a W row. Region kt (whose MFMAs read k-tile
// kt) forms k-tile kt + 1: rows 0..3 after the first 64 MFMAs' slots from
// data loaded half a region earlier, rows 4..7 after the last 64 from data
// loaded at the region's start. s_c and 1/s_c of a k-tile reach LDS by DMA
// a region ahead. About 13.5 VALU instructions per element (the transform's
// 12 plus the conversion of W and the packing) against the 2 that a
// 16x16x32 MFMA hides, so this kernel is bound by the VALU.
#include <utility>

#include "gemm_core.h"

namespace awq {
namespace {

__shared__ float sFuSI[2][128];   // per stage: s_c of the k-tile's 64 channels, then 1/s_c

struct FuCtx {
  __amdgpu_buffer_rsrc_t rsW, rsP, rsS, rsI;
  uint32_t wofs;       // bytes: lane's W entry (row 8j, channel 8kc) of k-tile 0
  uint32_t pofs;       // bytes: lane's parameter entry (row 8j) of group row 0
  uint32_t wrow, prow; // bytes per W row, per parameter row (K/G entries of 16 bytes)
  int kt_last, gshift;
  int lds[4];          // LDS byte offset within a stage of row 8j + r is lds[r / 2] + 128·r
  float qmax;
};

// Four rows' data for one k-tile: W's 8 channels and the row's group parameters.
struct FuHalf {
  uint4 w[4];
  float step[4], zero[4], rstep[4];
};

// first group row of k-tile kt for the wave (the lane's share at group size
// 32 is in pofs)
__device__ __forceinline__ uint32_t fu_group0(const FuCtx& f, int kt) {
  return f.gshift == 5 ? uint32_t(2 * kt) : uint32_t(kt) >> (f.gshift - 6);
}

// rows 4H .. 4H + 3 of k-tile kt (k-tiles past the end read the last one again)
template <int H>
__device__ __forceinline__ void fu_load(const FuCtx& f, int kt, FuHalf& h) {
  const int k = kt < f.kt_last ? kt : f.kt_last;
  const uint32_t g = fu_group0(f, k);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int R = 4 * H + r;
    const auto wv = __builtin_amdgcn_raw_buffer_load_b128(f.rsW, f.wofs,
                                                          int(R * f.wrow + uint32_t(k) * 128), 0);
    h.w[r] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    const auto pv = __builtin_amdgcn_raw_buffer_load_b96(f.rsP, f.pofs,
                                                         int(R * f.prow + g * 16), 0);
    h.step[r] = __uint_as_float(pv[0]);
    h.zero[r] = __uint_as_float(pv[1]);
    h.rstep[r] = __uint_as_float(pv[2]);
  }
}

// s_c and 1/s_c of k-tile kt into LDS stage kt % 2 (wave 0; 64 lanes x 4 bytes each)
__device__ __forceinline__ void fu_si_dma(const FuCtx& f, int kt, int wave) {
  if (wave != 0) return;
  const int k = kt < f.kt_last ? kt : f.kt_last;
  const int lane = threadIdx.x & 63;
  float* st = sFuSI[kt & 1];
  __builtin_amdgcn_raw_ptr_buffer_load_lds(f.rsS, AWQ_LDS(st), 4, lane * 4, k * 256, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(f.rsI, AWQ_LDS(st + 64), 4, lane * 4, k * 256, 0, 0);
}

__device__ __forceinline__ void fu_si_read(int kt, int kc, float (&sv)[8], float (&iv)[8]) {
  const float4* st = reinterpret_cast<const float4*>(sFuSI[kt & 1]);
  const float4 a = st[2 * kc], b = st[2 * kc + 1], c = st[16 + 2 * kc], d = st[17 + 2 * kc];
  sv[0] = a.x; sv[1] = a.y; sv[2] = a.z; sv[3] = a.w;
  sv[4] = b.x; sv[5] = b.y; sv[6] = b.z; sv[7] = b.w;
  iv[0] = c.x; iv[1] = c.y; iv[2] = c.z; iv[3] = c.w;
  iv[4] = d.x; iv[5] = d.y; iv[6] = d.z; iv[7] = d.w;
}

template <bool F16>
__device__ __forceinline__ float fu_w(uint32_t word, int hi) {
  if constexpr (F16) return f16_to_f32(uint16_t(hi ? word >> 16 : word & 0xFFFFu));
  else return __uint_as_float(hi ? word & 0xFFFF0000u : word << 16);
}

// Elements 4HH .. 4HH + 3 of row 4H + r: the transform's arithmetic; the
// row's 16-byte store after its second half.
template <bool F16, int S, int H, int r, int HH>
__device__ __forceinline__ void fu_form(const FuCtx& f, const FuHalf& h, const float (&sv)[8],
                                        const float (&iv)[8], uint32_t (&pk)[4]) {
#pragma clang fp contract(off)
  const uint32_t wa = HH ? h.w[r].z : h.w[r].x, wb = HH ? h.w[r].w : h.w[r].y;
  const QParams p{h.step[r], h.zero[r], f.qmax};
  float e[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int kk = 4 * HH + t;
    const float w = fu_w<F16>(t < 2 ? wa : wb, t & 1);
    const float qc = quant_code_centered(w * sv[kk], p, h.rstep[r]);
    e[t] = (qc * p.step) * iv[kk] - w;
  }
  // two values per packed conversion, each rounded to nearest even as the
  // transform's per-value conversion rounds it
  uint32_t lo, hi;
  if constexpr (F16) {
    asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(lo) : "v"(e[0]), "v"(e[1]));
    asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(hi) : "v"(e[2]), "v"(e[3]));
  } else {
    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(lo) : "v"(e[0]), "v"(e[1]));
    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(hi) : "v"(e[2]), "v"(e[3]));
  }
  pk[2 * HH] = lo;
  pk[2 * HH + 1] = hi;
  if constexpr (HH == 1) {
    constexpr int R = 4 * H + r;
    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(stage64_b<S>()) + f.lds[R / 2] + 128 * R) =
        make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
}

// MFMA m of region kt (stage S = kt % 2), then what follows it: after MFMA
// 8o + 1 of each half, element half o % 2 of row o / 2 of that half's rows;
// after MFMA 8o + 5 of the first half, X's DMA copy o of k-tile kt + 1.
template <bool F16, int S, bool PREV, int M, class V>
__device__ __forceinline__ void fu_slot(const GemmCtx64& c, const FuCtx& f, const int (&rdA)[2],
                                        const int (&rdB)[2], int kt, floatx4 (&acc)[8][8],
                                        V (&f0a)[8], V (&f0b)[8], V (&f1a)[8], V (&f1b)[8],
                                        const FuHalf& hA, const FuHalf& hB, const float (&sv)[8],
                                        const float (&iv)[8], uint32_t (&pk)[4]) {
  constexpr int u = (M % 64) / 4, t = M % 4, i = u >> 1, j = (u & 1) * 4 + t;
  if constexpr (M < 64) {
    if constexpr (PREV) mfma16(acc[i][j], f1a[i], f1b[j]);
    if constexpr (t == 0) frag16<S>(rdA[0], rdB[0], u, f0a, f0b);
  } else {
    mfma16_acc<!PREV>(acc[i][j], f0a[i], f0b[j]);
    if constexpr (t == 0) frag16<S>(rdA[1], rdB[1], u, f1a, f1b);
  }
  constexpr int o = (M % 64) / 8, e = M % 8;
  if constexpr (e == 1) {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (M < 64) fu_form<F16, S ^ 1, 0, o / 2, o % 2>(f, hA, sv, iv, pk);
    else fu_form<F16, S ^ 1, 1, o / 2, o % 2>(f, hB, sv, iv, pk);
    __builtin_amdgcn_sched_barrier(0);
  } else if constexpr (e == 5 && M < 64) {
    __builtin_amdgcn_sched_barrier(0);
    copy64<S ^ 1>(c, kt + 1, o);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <bool F16, int S, bool PREV, int OFF, class V, int... Ms>
__device__ __forceinline__ void fu_slots(const GemmCtx64& c, const FuCtx& f, const int (&rdA)[2],
                                         const int (&rdB)[2], int kt, floatx4 (&acc)[8][8],
                                         V (&f0a)[8], V (&f0b)[8], V (&f1a)[8], V (&f1b)[8],
                                         const FuHalf& hA, const FuHalf& hB,
                                         const float (&sv)[8], const float (&iv)[8],
                                         uint32_t (&pk)[4], std::integer_sequence<int, Ms...>) {
  (fu_slot<F16, S, PREV, OFF + Ms>(c, f, rdA, rdB, kt, acc, f0a, f0b, f1a, f1b, hA, hB, sv, iv,
                                   pk),
   ...);
}

// Region kt (stage S = kt % 2): rows 4..7 of k-tile kt + 1 and s_c, 1/s_c of
// k-tile kt + 2 are fetched first; rows 0..3 of k-tile kt + 2 between the
// two halves; one wait and one barrier at the end, as in gemm_core.h.
template <bool F16, int S, bool PREV, class V>
__device__ __forceinline__ void fu_region(const GemmCtx64& c, const FuCtx& f, const int (&rdA)[2],
                                          const int (&rdB)[2], int kt, int kc,
                                          floatx4 (&acc)[8][8], V (&f0a)[8], V (&f0b)[8],
                                          V (&f1a)[8], V (&f1b)[8], FuHalf& hA, FuHalf& hB) {
  fu_load<1>(f, kt + 1, hB);
  fu_si_dma(f, kt + 2, c.wave);
  float sv[8], iv[8];
  fu_si_read(kt + 1, kc, sv, iv);
  uint32_t pk[4];
  __builtin_amdgcn_sched_barrier(0);
  fu_slots<F16, S, PREV, 0>(c, f, rdA, rdB, kt, acc, f0a, f0b, f1a, f1b, hA, hB, sv, iv, pk,
                            std::make_integer_sequence<int, 64>{});
  __builtin_amdgcn_sched_barrier(0);
  fu_load<0>(f, kt + 2, hA);
  __builtin_amdgcn_sched_barrier(0);
  fu_slots<F16, S, PREV, 64>(c, f, rdA, rdB, kt, acc, f0a, f0b, f1a, f1b, hA, hB, sv, iv, pk,
                             std::make_integer_sequence<int, 64>{});
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  region_barrier();
}

template <bool F16>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void search_fused_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                         const float* __restrict__ P, const float* __restrict__ s_rows,
                         const float* __restrict__ inv_rows, int64_t s_stride, int64_t M,
                         int64_t N, int64_t K, int gshift, int bits, int tiles_m, int tiles_n,
                         float* __restrict__ partials) {
  typedef typename Operand<F16>::type V;
  int tm, tn;
  if (!tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;   // n0: row of the stacked E
  const int64_t rows_a = M - m0 < BM ? M - m0 : BM;
  const int64_t cand = n0 / N, nr = n0 % N;   // N is a multiple of 256: one candidate per tile
  const int tid = threadIdx.x;
  GemmCtx64 c;
  gemm_setup64(c, X + m0 * K, rows_a, X + m0 * K, rows_a, K);
  FuCtx f;
  const int64_t KG = K >> gshift;
  f.rsW = tile_rsrc(W + nr * K, BN, K);
  f.rsP = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(P + (cand * N + nr) * KG * 4), 0,
                                            int(BN * KG * 16), 0x00020000);
  f.rsS = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(s_rows + cand * s_stride), 0,
                                            int(K * 4), 0x00020000);
  f.rsI = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(inv_rows + cand * s_stride), 0,
                                            int(K * 4), 0x00020000);
  const int j = tid >> 3, kc = tid & 7;
  f.wrow = uint32_t(K * 2);
  f.prow = uint32_t(KG * 16);
  f.wofs = uint32_t(8 * j) * f.wrow + uint32_t(kc) * 16;
  // at group size 32 the lane's channels 8kc .. 8kc + 7 sit in the k-tile's
  // second group for kc >= 4
  f.pofs = uint32_t(8 * j) * f.prow + (gshift == 5 ? uint32_t(kc >> 2) * 16 : 0u);
  f.kt_last = int(K / 64) - 1;
  f.gshift = gshift;
  f.qmax = float((1 << bits) - 1);
#pragma unroll
  for (int t = 0; t < 4; ++t) f.lds[t] = 1024 * j + 16 * ((kc ^ (4 * (j & 1))) ^ t);

  int rdA[2], rdB[2];
  frag_offsets16(c, rdA, rdB);
  floatx4 acc[8][8];
  // prologue: s_c, 1/s_c of k-tiles 0 and 1; k-tile 0 of X and of the
  // operand in stage 0; rows 0..3 of k-tile 1, which region 0 forms first
  FuHalf hA, hB;
  fu_si_dma(f, 0, c.wave);
  fu_si_dma(f, 1, c.wave);
  fu_load<0>(f, 0, hA);
  fu_load<1>(f, 0, hB);
  dma64_a<0>(c, 0);
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  region_barrier();
  {
    float sv[8], iv[8];
    fu_si_read(0, kc, sv, iv);
    uint32_t pk[4];
    fu_form<F16, 0, 0, 0, 0>(f, hA, sv, iv, pk); fu_form<F16, 0, 0, 0, 1>(f, hA, sv, iv, pk);
    fu_form<F16, 0, 0, 1, 0>(f, hA, sv, iv, pk); fu_form<F16, 0, 0, 1, 1>(f, hA, sv, iv, pk);
    fu_form<F16, 0, 0, 2, 0>(f, hA, sv, iv, pk); fu_form<F16, 0, 0, 2, 1>(f, hA, sv, iv, pk);
    fu_form<F16, 0, 0, 3, 0>(f, hA, sv, iv, pk); fu_form<F16, 0, 0, 3, 1>(f, hA, sv, iv, pk);
    fu_form<F16, 0, 1, 0, 0>(f, hB, sv, iv, pk); fu_form<F16, 0, 1, 0, 1>(f, hB, sv, iv, pk);
    fu_form<F16, 0, 1, 1, 0>(f, hB, sv, iv, pk); fu_form<F16, 0, 1, 1, 1>(f, hB, sv, iv, pk);
    fu_form<F16, 0, 1, 2, 0>(f, hB, sv, iv, pk); fu_form<F16, 0, 1, 2, 1>(f, hB, sv, iv, pk);
    fu_form<F16, 0, 1, 3, 0>(f, hB, sv, iv, pk); fu_form<F16, 0, 1, 3, 1>(f, hB, sv, iv, pk);
  }
  fu_load<0>(f, 1, hA);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  region_barrier();
  V f0a[8], f0b[8], f1a[8], f1b[8];
  fu_region<F16, 0, false>(c, f, rdA, rdB, 0, kc, acc, f0a, f0b, f1a, f1b, hA, hB);
  int kt = 1;
  for (; kt + 1 < c.KT; kt += 2) {
    fu_region<F16, 1, true>(c, f, rdA, rdB, kt, kc, acc, f0a, f0b, f1a, f1b, hA, hB);
    fu_region<F16, 0, true>(c, f, rdA, rdB, kt + 1, kc, acc, f0a, f0b, f1a, f1b, hA, hB);
  }
  if (kt < c.KT) fu_region<F16, 1, true>(c, f, rdA, rdB, kt, kc, acc, f0a, f0b, f1a, f1b, hA, hB);
  mfma_8x8(acc, f1a, f1b);
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) asm volatile("" : "+a"(acc[i][jj]));

  // epilogue of the search GEMM: the squares summed per output column
  const int lane = tid & 63;
  const int wm = c.wave >> 1, wn = c.wave & 1;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float* red = reinterpret_cast<float*>(s64A0);  // [2][BN]
  column_square_sums(acc, red, wm, wn, lane);
  __syncthreads();
  const int64_t Nc = int64_t(tiles_n) * BN;
  partials[int64_t(tm) * Nc + n0 + tid] = red[tid] + red[BN + tid];
}

}  // namespace

// One launch over all candidates of a batch: nc·N stacked rows, N a multiple
// of 256, K of 128, group 32, 64 or 128; P from launch_group_params with
// cand_stride N·K/G.
hipError_t launch_search_fused(const void* X, int dtype, const void* W, const float* P,
                               const float* s_rows, const float* inv_rows, int64_t s_stride,
                               int64_t M, int64_t N, int64_t K, int nc, int group, int bits,
                               float* partials, hipStream_t st) {
  if ((dtype != 1 && dtype != 2) || N % BN || K % 128 ||
      (group != 32 && group != 64 && group != 128))
    return hipErrorInvalidValue;
  const int gshift = group == 32 ? 5 : group == 64 ? 6 : 7;
  const int tiles_m = int((M + BM - 1) / BM), tiles_n = int(int64_t(nc) * N / BN);
  const unsigned blocks = unsigned(gemm_blocks(tiles_m, tiles_n));
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const uint16_t* w = static_cast<const uint16_t*>(W);
  if (dtype == 2)
    search_fused_kernel<true><<<blocks, NT, 0, st>>>(x, w, P, s_rows, inv_rows, s_stride, M, N,
                                                     K, gshift, bits, tiles_m, tiles_n, partials);
  else
    search_fused_kernel<false><<<blocks, NT, 0, st>>>(x, w, P, s_rows, inv_rows, s_stride, M, N,
                                                      K, gshift, bits, tiles_m, tiles_n, partials);
  return hipGetLastError();
}

}  // namespace awq
