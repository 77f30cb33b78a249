// The MFMA main loop of the search GEMM (sums of squares of X·Eᵀ), the
// Gram build and search, and the W4A16 consumer's prefill GEMM (X·Ŵᵀ
// stored): a 256x256 output tile per workgroup, A and B both [rows, K]
// row-major 16-bit operands.
//
//  * 256x256 block tile, four wavefronts (one per SIMD) in a 2x2 arrangement,
//    each owning 128x128 outputs as 8x8 blocks of v_mfma_f32_16x16x32
//    accumulators (bf16 or fp16 operands, 256 AGPRs). On random data the
//    16x16x32 form sustains a higher rate than 32x32x16 under the chip's
//    power limit. Its accumulators are pinned to AGPRs through inline asm
//    (gemm_mainloop16, below).
//  * K advances in 64-wide k-tiles through a 2-stage LDS ring (2 x 64 KiB)
//    filled by buffer_load_dwordx4 ... lds (no staging registers). Loads go
//    through a buffer resource per tile, so rows past the end of A or B read
//    as zero. One k-tile per barrier-delimited region.
//  * Each LDS stage is its own __shared__ array and the k-loop is unrolled
//    over the stages, so the compiler can tell the stage being read from the
//    stage the DMA writes and does not serialise LDS reads behind the DMA.
//  * Workgroups are mapped so each XCD runs 4 A tiles x 8 B tiles at a time
//    while all XCDs share the same 8 B tiles.
//
// Output layout of one 16x16 accumulator: lane l holds column l % 16; its
// register v holds row 4·(l / 16) + v.
#pragma once

#include "device_common.h"

namespace awq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// MFMA operand vector of 8 elements: bf16 or fp16 (F16 = true).
template <bool F16>
struct Operand {
  typedef bf16x8_t type;
};
template <>
struct Operand<true> {
  typedef f16x8_t type;
};

#define AWQ_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int NT = 256;

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int wait_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xF | (3 << 14) | (0x7 << 4);

// Masks for __builtin_amdgcn_sched_group_barrier.
constexpr int kSgValu = 0x002, kSgMfma = 0x008, kSgVmemRead = 0x020, kSgDsRead = 0x100,
              kSgDsWrite = 0x200;

// Workgroup barrier that neither the compiler nor the scheduler may move a
// memory operation or any instruction across. Unlike __syncthreads() it adds
// no vmcnt(0), so DMA copies stay in flight across it.
__device__ __forceinline__ void region_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Block id -> (token tile, candidate-column tile). Returns false for padding
// blocks. Every 256 consecutive ids give each XCD 4 token tiles x 8 column
// tiles (consecutive ids go round-robin over the 8 XCDs). From 32 token tiles
// on, all XCDs take the same 8 column tiles and 32 token tiles between them;
// with 16, 8 or 4 token tiles (4096, 2048, 1024 tokens) the 8 XCDs split
// into 4, 2 or 1 token groups x 2, 4 or 8 column groups.
__device__ __forceinline__ bool tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  if (tiles_m >= 32) {
    const int w = bid >> 8, j = bid & 255;
    const int xcd = j & 7, i = j >> 3;
    const int nwn = (tiles_n + 7) >> 3;
    const int g = w / nwn, wn = w - g * nwn;
    tm = 32 * g + 4 * xcd + (i & 3);
    tn = 8 * wn + (i >> 2);
  } else if (tiles_m == 16 || tiles_m == 8 || tiles_m == 4) {
    const int w = bid >> 8, j = bid & 255;
    const int xcd = j & 7, i = j >> 3;
    const int nag = tiles_m >> 2;                 // token groups of 4 tiles
    const int ag = xcd & (nag - 1), bg = (8 / nag) * w + xcd / nag;
    tm = 4 * ag + (i & 3);
    tn = 8 * bg + (i >> 2);
  } else {
    tm = bid % tiles_m;
    tn = bid / tiles_m;
  }
  return tm < tiles_m && tn < tiles_n;
}

// Buffer resource over `rows` rows of K bf16 starting at `base` (dword 3 =
// raw 32-bit data format, the gfx9-family default). Offsets past the end
// read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int64_t rows,
                                                           int64_t K) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0,
                                           int(rows * K * 2), 0x00020000);
}

// The 2-stage ring of 64-wide k-tiles (2 x 64 KiB). Each region (one k-tile)
// issues the DMA of k-tile kt + 1 into the other stage (last read in region
// kt - 1), runs the MFMAs of the previous k-step while the next fragments
// are read, and ends with one wait (this wave's LDS reads and its DMA of
// kt + 1) and one barrier. LDS rows are 128 bytes (8 chunks of 16 B) with
// the chunk index XORed by (row / 2) % 8, which keeps a 16-lane fragment
// read on 16 distinct bank groups and lets the DMA fill whole rows.
constexpr int BK64 = 64;
constexpr int CH64 = 8;
constexpr int STAGE64 = 256 * CH64;
__shared__ uint4 s64A0[STAGE64], s64A1[STAGE64], s64B0[STAGE64], s64B1[STAGE64];
template <int S>
__device__ __forceinline__ uint4* stage64_a() { return S == 0 ? s64A0 : s64A1; }
template <int S>
__device__ __forceinline__ uint4* stage64_b() { return S == 0 ? s64B0 : s64B1; }
__device__ __forceinline__ int swz64(int row, int chunk) {
  return row * CH64 + (chunk ^ ((row >> 1) & 7));
}
// A and B with their own row strides (elements). With pair_b, A's
// contraction alternates 128-wide blocks P_0, Q_0, P_1, Q_1, ... and each
// 128-wide block of B is read twice in a row, so one k-loop gives
// Σ_c (P_c + Q_c)·B_cᵀ: A's 64-wide k-tile kt reads B's k-tile
// (kt / 4)·2 + kt % 2. pair_a is the same with the roles swapped: B
// alternates P_c, Q_c and each 128-wide block of A is read twice.
// Copy j of a wave fills rows 8·j further down than copy 0, so its source
// offset is a per-lane base (two of them: the swizzle flips by 4 on odd j)
// plus a uniform step j·8·ld·2 bytes, which goes in the scalar offset.
// rev: the k-loop visits the k-tiles from the last to the first (the
// accumulation order changes, the pairing does not), so that loops of
// different lengths over the same operand's tail read the same k-tiles at
// the same time.
struct GemmCtx64 {
  __amdgpu_buffer_rsrc_t rsA, rsB;
  int vbaseA[2], vbaseB[2];
  int stepA, stepB;
  int wave, KT, oobA, oobB;
  bool pair_a, pair_b, rev;
};
__device__ __forceinline__ void gemm_setup64(GemmCtx64& c, const uint16_t* A, int64_t rows_a,
                                             int64_t lda, const uint16_t* B, int64_t rows_b,
                                             int64_t ldb, int64_t KA, bool pair_b,
                                             bool pair_a = false) {
  c.rsA = tile_rsrc(A, rows_a, lda);
  c.rsB = tile_rsrc(B, rows_b, ldb);
  const int tid = threadIdx.x, lane = tid & 63;
  c.wave = tid >> 6;
  c.KT = int(KA / BK64);
  c.pair_a = pair_a;
  c.pair_b = pair_b;
  c.rev = false;
  c.oobA = BM * int(lda) * 2;
  c.oobB = BN * int(ldb) * 2;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = (c.wave * 8 + j) * 64 + lane;
    const int row = p >> 3;
    const int chunk = (p & 7) ^ ((row >> 1) & 7);
    c.vbaseA[j] = ((row - 8 * j) * int(lda) + chunk * 8) * 2;
    c.vbaseB[j] = ((row - 8 * j) * int(ldb) + chunk * 8) * 2;
  }
  c.stepA = 16 * int(lda);
  c.stepB = 16 * int(ldb);
}
__device__ __forceinline__ void gemm_setup64(GemmCtx64& c, const uint16_t* A, int64_t rows_a,
                                             const uint16_t* B, int64_t rows_b, int64_t K) {
  gemm_setup64(c, A, rows_a, K, B, rows_b, K, K, false);
}
template <int S>
__device__ __forceinline__ void dma64(const GemmCtx64& c, int kt) {
  const bool in = kt < c.KT;
  if (c.rev && in) kt = c.KT - 1 - kt;
  const int kta = c.pair_a ? ((kt >> 2) << 1) | (kt & 1) : kt;
  const int ktb = c.pair_b ? ((kt >> 2) << 1) | (kt & 1) : kt;
  const int kofsA = in ? kta * (BK64 * 2) : c.oobA;
  const int kofsB = in ? ktb * (BK64 * 2) : c.oobB;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsA, AWQ_LDS(stage64_a<S>() + (c.wave * 8 + j) * 64),
                                             16, c.vbaseA[j & 1] + kofsA, j * c.stepA, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsB, AWQ_LDS(stage64_b<S>() + (c.wave * 8 + j) * 64),
                                             16, c.vbaseB[j & 1] + kofsB, j * c.stepB, 0, 0);
  }
}
// 8x8 blocks of 16x16x32 MFMAs per wave.
// The accumulators are pinned to AGPRs through inline asm (the builtin form
// makes the register allocator shuttle 4-register tuples inside the loop).
// The asm is volatile, so LDS reads and copies keep their source order
// around it: the interleaving below is written out instead of requested
// with scheduling groups. The compiler inserts no hazard waits around asm,
// so no VALU instruction may touch the accumulators near an MFMA: the first
// MFMA of each accumulator takes the constant 0 as its addend (no zeroing
// moves), and the loop ends with an explicit wait tied to every
// accumulator before anything reads them.
typedef float floatx4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void mfma16(floatx4& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16(floatx4& c, const f16x8_t& a, const f16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_first(floatx4& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_first(floatx4& c, const f16x8_t& a, const f16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
}
template <bool FIRST, class V>
__device__ __forceinline__ void mfma16_acc(floatx4& c, const V& a, const V& b) {
  if (FIRST) mfma16_first(c, a, b);
  else mfma16(c, a, b);
}
// lane l supplies row l % 16 of a block and k 8·(l / 16) .. +7 of the
// 32-wide k-step ks (chunk 4·ks + l / 16); block i is 16 rows further on,
// which leaves the (row / 2) % 8 swizzle unchanged
__device__ __forceinline__ void frag_offsets16(const GemmCtx64& c, int (&rdA)[2], int (&rdB)[2]) {
  const int lane = threadIdx.x & 63;
  const int wm = c.wave >> 1, wn = c.wave & 1;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    rdA[ks] = swz64(wm * 128 + (lane & 15), 4 * ks + (lane >> 4));
    rdB[ks] = swz64(wn * 128 + (lane & 15), 4 * ks + (lane >> 4));
  }
}
template <int S, class V>
__device__ __forceinline__ void frag16(int rdA, int rdB, int r, V (&fa)[8], V (&fb)[8]) {
  // fragment read r of a k-step: B blocks first (the first MFMA row needs
  // all of them), then A blocks
  if (r < 8) fb[r] = __builtin_bit_cast(V, stage64_b<S>()[rdB + r * 128]);
  else fa[r - 8] = __builtin_bit_cast(V, stage64_a<S>()[rdA + (r - 8) * 128]);
}
template <int S>
__device__ __forceinline__ void copy64(const GemmCtx64& c, int kt, int q) {
  // copy q of the 16 a wave issues per k-tile: A rows for q < 8, then B
  const bool in = kt < c.KT;
  if (c.rev && in) kt = c.KT - 1 - kt;
  const int j = q & 7;
  if (q < 8) {
    const int kta = c.pair_a ? ((kt >> 2) << 1) | (kt & 1) : kt;
    const int kofsA = in ? kta * (BK64 * 2) : c.oobA;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsA, AWQ_LDS(stage64_a<S>() + (c.wave * 8 + j) * 64),
                                             16, c.vbaseA[j & 1] + kofsA, j * c.stepA, 0, 0);
  } else {
    const int ktb = c.pair_b ? ((kt >> 2) << 1) | (kt & 1) : kt;
    const int kofsB = in ? ktb * (BK64 * 2) : c.oobB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsB, AWQ_LDS(stage64_b<S>() + (c.wave * 8 + j) * 64),
                                             16, c.vbaseB[j & 1] + kofsB, j * c.stepB, 0, 0);
  }
}
// Only A's copies of k-tile kt (for loops whose B operand is formed in
// registers).
template <int S>
__device__ __forceinline__ void dma64_a(const GemmCtx64& c, int kt) {
#pragma unroll
  for (int q = 0; q < 8; ++q) copy64<S>(c, kt, q);
}
// One k-tile: the previous k-step's 64 MFMAs (f1) carry k-step 0's 16
// fragment reads and the next k-tile's 16 copies, one each per four MFMAs;
// k-step 0's MFMAs (f0) carry k-step 1's reads, one per four MFMAs.
// NEXT: the copies fetch k-tile 0 of another tile (context cn) instead of
// k-tile kt + 1 of this one.
template <int S, bool PREV, bool NEXT = false, class V>
__device__ __forceinline__ void region16(const GemmCtx64& c, const int (&rdA)[2], const int (&rdB)[2],
                                         int kt, floatx4 (&acc)[8][8], V (&f0a)[8], V (&f0b)[8],
                                         V (&f1a)[8], V (&f1b)[8], const GemmCtx64* cn = nullptr) {
  const GemmCtx64& cc = NEXT ? *cn : c;
  const int ktc = NEXT ? 0 : kt + 1;
  if (PREV) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int i = q >> 1, j0 = (q & 1) * 4;
      mfma16(acc[i][j0], f1a[i], f1b[j0]);
      frag16<S>(rdA[0], rdB[0], q, f0a, f0b);
      mfma16(acc[i][j0 + 1], f1a[i], f1b[j0 + 1]);
      mfma16(acc[i][j0 + 2], f1a[i], f1b[j0 + 2]);
      copy64<S ^ 1>(cc, ktc, q);
      mfma16(acc[i][j0 + 3], f1a[i], f1b[j0 + 3]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q) copy64<S ^ 1>(cc, ktc, q);
#pragma unroll
    for (int q = 0; q < 16; ++q) frag16<S>(rdA[0], rdB[0], q, f0a, f0b);
  }
  // without PREV this is the first k-step: each accumulator starts here
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = q >> 1, j0 = (q & 1) * 4;
    mfma16_acc<!PREV>(acc[i][j0], f0a[i], f0b[j0]);
    frag16<S>(rdA[1], rdB[1], q, f1a, f1b);
    mfma16_acc<!PREV>(acc[i][j0 + 1], f0a[i], f0b[j0 + 1]);
    mfma16_acc<!PREV>(acc[i][j0 + 2], f0a[i], f0b[j0 + 2]);
    mfma16_acc<!PREV>(acc[i][j0 + 3], f0a[i], f0b[j0 + 3]);
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  region_barrier();
}
template <class V>
__device__ __forceinline__ void mfma_8x8(floatx4 (&acc)[8][8], const V (&fa)[8], const V (&fb)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) mfma16(acc[i][j], fa[i], fb[j]);
}
// Writes every accumulator (no zeroing needed by the caller) and ends with
// them safe to read (the last MFMAs have drained).
template <bool F16>
__device__ __forceinline__ void gemm_mainloop16(const GemmCtx64& c, floatx4 (&acc)[8][8]) {
  typedef typename Operand<F16>::type V;
  int rdA[2], rdB[2];
  frag_offsets16(c, rdA, rdB);
  dma64<0>(c, 0);
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  region_barrier();
  V f0a[8], f0b[8], f1a[8], f1b[8];
  region16<0, false>(c, rdA, rdB, 0, acc, f0a, f0b, f1a, f1b);
  int kt = 1;
  for (; kt + 1 < c.KT; kt += 2) {
    region16<1, true>(c, rdA, rdB, kt, acc, f0a, f0b, f1a, f1b);
    region16<0, true>(c, rdA, rdB, kt + 1, acc, f0a, f0b, f1a, f1b);
  }
  if (kt < c.KT) {
    region16<1, true>(c, rdA, rdB, kt, acc, f0a, f0b, f1a, f1b);
  }
  mfma_8x8(acc, f1a, f1b);
  // the compiler sees no MFMA in the asm, so it inserts no wait before the
  // accumulators are read; the empty statements tie every read to the nops
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// The k-loop of one tile in a chain of tiles: k-tile 0 is already in stage
// 0 (copied by the previous tile's last region, or by the caller before the
// first tile), KT is even and at least 2, and the last region copies k-tile
// 0 of the next tile (context cn) into stage 0. Same accumulator contract
// as gemm_mainloop16.
template <bool F16>
__device__ __forceinline__ void gemm_mainloop16_chain(const GemmCtx64& c, const GemmCtx64& cn,
                                                      floatx4 (&acc)[8][8]) {
  typedef typename Operand<F16>::type V;
  int rdA[2], rdB[2];
  frag_offsets16(c, rdA, rdB);
  V f0a[8], f0b[8], f1a[8], f1b[8];
  region16<0, false>(c, rdA, rdB, 0, acc, f0a, f0b, f1a, f1b);
  int kt = 1;
  for (; kt + 2 < c.KT; kt += 2) {
    region16<1, true>(c, rdA, rdB, kt, acc, f0a, f0b, f1a, f1b);
    region16<0, true>(c, rdA, rdB, kt + 1, acc, f0a, f0b, f1a, f1b);
  }
  region16<1, true, true>(c, rdA, rdB, kt, acc, f0a, f0b, f1a, f1b, &cn);
  mfma_8x8(acc, f1a, f1b);
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// Epilogue of the search GEMMs: each lane's 4 accumulators of block (i, j)
// lie in output column j·16 + lane % 16 of the wave's 128 columns, and lanes
// l, l^16, l^32, l^48 share that column. The squares are summed over the
// wave's 128 rows (one FMA each, rows in block order) and the result goes to
// red[wm·BN + wn·128 + column].
__device__ __forceinline__ void column_square_sums(const floatx4 (&acc)[8][8], float* red, int wm,
                                                   int wn, int lane) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) s = __builtin_fmaf(acc[i][j][v], acc[i][j][v], s);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (lane < 16) red[wm * BN + wn * 128 + j * 16 + lane] = s;
  }
}

// Number of workgroups the tile_of mapping needs for a tiles_m x tiles_n grid.
__host__ __device__ inline int64_t gemm_blocks(int tiles_m, int tiles_n) {
  if (tiles_m >= 32) return int64_t((tiles_m + 31) / 32) * 32 * (int64_t((tiles_n + 7) / 8) * 8);
  if (tiles_m == 16 || tiles_m == 8 || tiles_m == 4) {
    const int per = 64 / (tiles_m >> 2);           // column tiles per 256 ids
    return int64_t((tiles_n + per - 1) / per) * 256;
  }
  return int64_t(tiles_m) * tiles_n;
}

}  // namespace
}  // namespace awq
