// Consumer of the packed layout: a weight-only INT4 linear layer with 16-bit
// activations (W4A16),
//
//   Y[t][n] = Σ_k X'[t][k] · Ŵ[n][k],   Ŵ[n][k] = (q[k][n] - z[k/g][n]) · scale[k/g][n]
//
// where X' = X·diag(s)^-1 is what the folded preceding operation produces and
// (q, z, scale) is the layout the pack kernel writes ("05 — AWQ", section 5
// "Bit-level output format": qweight [K, N/8], qzeros [K/g, N/8], fp16
// scales [K/g, N]; the reading note's "Key takeaways": weight-only 4-bit with
// 16-bit activations). Ŵ is formed exactly in float32 ((q - z) is an integer
// of at most 4 bits and the scale an fp16 value).
//
// Four kernels, by the number of token rows T and the layout:
//  * T <= 16 (decode), N a multiple of 16: the codes go to the matrix cores
//    as exact small numbers (B = 1 + q/16) against the activations, 16 token
//    rows per v_mfma_f32_16x16x32, and the zero points and scales are applied
//    to the float32 block sums (w4a16_mgemv_kernel, below; also for the
//    3-bit layout, whose codes a lane pair funnel-shifts into place).
//  * T <= 16 otherwise: fused float32 GEMV. A lane owns one qweight word
//    column (8 output channels) and a run of k rows; it dequantises each word
//    in registers and accumulates T x 8 float32 sums.
//    In both, the 4 waves of a workgroup take consecutive k runs and meet in
//    LDS; one float32 partial per (k chunk, t, n) goes to the workspace and a
//    second kernel adds the chunks in a fixed order and rounds once to the
//    output type. Bound by HBM reads of qweight (N·K/2 bytes) and by the
//    unpacking ALU work.
//  * T > 16 (prefill): the packed layer is dequantised once into [N, K]
//    16-bit operand rows in the workspace (rounded once, to nearest even, to
//    the activation type), then the MFMA main loop of the search GEMM
//    (gemm_core.h) computes X'·Ŵᵀ and the epilogue rounds each float32 sum
//    once to the output type. At T = 4096 the extra pass moves N·K·2.5 bytes,
//    a few per cent of the GEMM's time.
//  * T > 16, 4 bits, on request: the same main loop with the B operand
//    formed from the packed layer in registers (w4a16_gemm_q_kernel, no
//    workspace), bit for bit the operand of the dequantisation pass. One
//    wave both feeds its matrix core and does the unpacking, so its VALU
//    work sits between the MFMAs; at T = 4096 it runs behind the two-pass
//    path.
#include <utility>

#include "gemm_core.h"

namespace awq {
namespace {

template <bool F16>
__device__ __forceinline__ uint16_t to16(float f) {
  if constexpr (F16) return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  else return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <bool F16>
__device__ __forceinline__ float from16(uint16_t h) {
  if constexpr (F16) return f16_to_f32(h);
  else return bf16_to_f32(h);
}

// The 8 fp16 scales of output channels 8j..8j+7 in group g (16 bytes) and
// their 8 zero points (one packed word) as float32.
__device__ __forceinline__ void group_params(const int32_t* __restrict__ qzeros,
                                             const uint16_t* __restrict__ scales, int64_t N,
                                             int64_t g, int64_t j, float (&sc)[8],
                                             float (&zf)[8]) {
  const uint4 s4 = *reinterpret_cast<const uint4*>(scales + g * N + 8 * j);
  const uint32_t sw[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[2 * i] = f16_to_f32(uint16_t(sw[i] & 0xFFFFu));
    sc[2 * i + 1] = f16_to_f32(uint16_t(sw[i] >> 16));
  }
  const uint32_t zw = uint32_t(qzeros[g * (N / 8) + j]);
#pragma unroll
  for (int r = 0; r < 8; ++r) zf[r] = float((zw >> (4 * r)) & 0xFu);
}

// ---------------------------------------------------------------------------
// prefill: dequantise into [N, K] operand rows
// ---------------------------------------------------------------------------

// Lane (kb, j): k rows 8kb..8kb+7 of word column j -> 8 output rows x 8 k,
// one 16-byte store per output row (consecutive lanes continue the same row).
template <bool F16>
__global__ __launch_bounds__(256) void dequant_kernel(const int32_t* __restrict__ qweight,
                                                      const int32_t* __restrict__ qzeros,
                                                      const uint16_t* __restrict__ scales,
                                                      int64_t N, int64_t K, int group,
                                                      uint16_t* __restrict__ Wd) {
#pragma clang fp contract(off)
  const int64_t K8 = K / 8, N8 = N / 8;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= K8 * N8) return;
  const int64_t kb = t % K8, j = t / K8;
  const int64_t k0 = kb * 8;
  float sc[8], zf[8];
  group_params(qzeros, scales, N, k0 / group, j, sc, zf);
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = uint32_t(qweight[(k0 + i) * N8 + j]);
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = (float((w[2 * i] >> (4 * r)) & 0xFu) - zf[r]) * sc[r];
      const float hi = (float((w[2 * i + 1] >> (4 * r)) & 0xFu) - zf[r]) * sc[r];
      h[i] = uint32_t(to16<F16>(lo)) | (uint32_t(to16<F16>(hi)) << 16);
    }
    *reinterpret_cast<uint4*>(Wd + (8 * j + r) * K + k0) = make_uint4(h[0], h[1], h[2], h[3]);
  }
}

// N a multiple of 32: lane (kb, j) takes k rows 8kb..8kb+7 of word columns
// 4j..4j+3 (output rows 32j..32j+31) with one 16-byte load per k row, so a
// 128-byte line of qweight feeds 8 lanes instead of 32.
template <bool F16>
__global__ __launch_bounds__(256) void dequant4x4_kernel(const int32_t* __restrict__ qweight,
                                                         const int32_t* __restrict__ qzeros,
                                                         const uint16_t* __restrict__ scales,
                                                         int64_t N, int64_t K, int group,
                                                         uint16_t* __restrict__ Wd) {
#pragma clang fp contract(off)
  const int64_t K8 = K / 8, N8 = N / 8, N32 = N / 32;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= K8 * N32) return;
  const int64_t kb = t % K8, j = t / K8;
  const int64_t k0 = kb * 8, g = k0 / group;
  uint4 w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = *reinterpret_cast<const uint4*>(qweight + (k0 + i) * N8 + 4 * j);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float sc[8], zf[8];
    group_params(qzeros, scales, N, g, 4 * j + c, sc, zf);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a = c == 0 ? w[2 * i].x : c == 1 ? w[2 * i].y : c == 2 ? w[2 * i].z : w[2 * i].w;
        const uint32_t b = c == 0 ? w[2 * i + 1].x : c == 1 ? w[2 * i + 1].y
                         : c == 2 ? w[2 * i + 1].z : w[2 * i + 1].w;
        const float lo = (float((a >> (4 * r)) & 0xFu) - zf[r]) * sc[r];
        const float hi = (float((b >> (4 * r)) & 0xFu) - zf[r]) * sc[r];
        h[i] = uint32_t(to16<F16>(lo)) | (uint32_t(to16<F16>(hi)) << 16);
      }
      *reinterpret_cast<uint4*>(Wd + (32 * j + 8 * c + r) * K + k0) =
          make_uint4(h[0], h[1], h[2], h[3]);
    }
  }
}

// 3-bit codes: row k of qweight holds the N codes densely, code n in bits
// 3n .. 3n+2 of the row's little-endian word stream, so 32 codes fill 3 words
// and codes 10 and 21 of each 32 straddle two words (zero points the same).
template <int R>
__device__ __forceinline__ uint32_t code3(const uint32_t (&w)[3]) {
  constexpr int bit = 3 * R, wi = bit / 32, sh = bit % 32;
  uint32_t v = w[wi] >> sh;
  if constexpr (sh > 29) v |= w[wi + 1] << (32 - sh);
  return v & 7u;
}

// Lane (kb, j): k rows 8kb..8kb+7 of output rows 32j..32j+31 (3 words per k
// row); one 16-byte store of 8 k per output row, consecutive lanes continuing
// the same row. Ŵ = (q - z)·scale in float32, rounded once to the 16-bit type.
template <bool F16>
__global__ __launch_bounds__(256) void dequant3_kernel(const int32_t* __restrict__ qweight,
                                                       const int32_t* __restrict__ qzeros,
                                                       const uint16_t* __restrict__ scales,
                                                       int64_t N, int64_t K, int group,
                                                       uint16_t* __restrict__ Wd) {
#pragma clang fp contract(off)
  const int64_t K8 = K / 8, N32 = N / 32, W3 = N / 32 * 3;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= K8 * N32) return;
  const int64_t kb = t % K8, j = t / K8;
  const int64_t k0 = kb * 8, g = k0 / group;
  uint32_t zw[3], w[8][3];
#pragma unroll
  for (int i = 0; i < 3; ++i) zw[i] = uint32_t(qzeros[g * W3 + 3 * j + i]);
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int i = 0; i < 3; ++i) w[e][i] = uint32_t(qweight[(k0 + e) * W3 + 3 * j + i]);
  const uint16_t* sg = scales + g * N + 32 * j;
#define AWQ_DQ3_ROW(R)                                                                        \
  {                                                                                           \
    const float zf = float(code3<R>(zw));                                                     \
    const float sc = f16_to_f32(sg[R]);                                                       \
    uint32_t h[4];                                                                            \
    for (int i = 0; i < 4; ++i) {                                                             \
      const float lo = (float(code3<R>(w[2 * i])) - zf) * sc;                                 \
      const float hi = (float(code3<R>(w[2 * i + 1])) - zf) * sc;                             \
      h[i] = uint32_t(to16<F16>(lo)) | (uint32_t(to16<F16>(hi)) << 16);                       \
    }                                                                                         \
    *reinterpret_cast<uint4*>(Wd + (32 * j + R) * K + k0) = make_uint4(h[0], h[1], h[2], h[3]); \
  }
  AWQ_DQ3_ROW(0) AWQ_DQ3_ROW(1) AWQ_DQ3_ROW(2) AWQ_DQ3_ROW(3) AWQ_DQ3_ROW(4) AWQ_DQ3_ROW(5)
  AWQ_DQ3_ROW(6) AWQ_DQ3_ROW(7) AWQ_DQ3_ROW(8) AWQ_DQ3_ROW(9) AWQ_DQ3_ROW(10) AWQ_DQ3_ROW(11)
  AWQ_DQ3_ROW(12) AWQ_DQ3_ROW(13) AWQ_DQ3_ROW(14) AWQ_DQ3_ROW(15) AWQ_DQ3_ROW(16)
  AWQ_DQ3_ROW(17) AWQ_DQ3_ROW(18) AWQ_DQ3_ROW(19) AWQ_DQ3_ROW(20) AWQ_DQ3_ROW(21)
  AWQ_DQ3_ROW(22) AWQ_DQ3_ROW(23) AWQ_DQ3_ROW(24) AWQ_DQ3_ROW(25) AWQ_DQ3_ROW(26)
  AWQ_DQ3_ROW(27) AWQ_DQ3_ROW(28) AWQ_DQ3_ROW(29) AWQ_DQ3_ROW(30) AWQ_DQ3_ROW(31)
#undef AWQ_DQ3_ROW
}

// ---------------------------------------------------------------------------
// prefill: MFMA GEMM with a store epilogue
// ---------------------------------------------------------------------------

template <bool F16>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void w4a16_gemm_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wd,
                       int64_t M, int64_t N, int64_t K, int tiles_m, int tiles_n,
                       uint16_t* __restrict__ Y) {
  int tm, tn;
  if (!tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;
  const int64_t rows_a = M - m0 < BM ? M - m0 : BM;
  const int64_t rows_b = N - n0 < BN ? N - n0 : BN;
  GemmCtx64 c;
  gemm_setup64(c, X + m0 * K, rows_a, Wd + n0 * K, rows_b, K);
  floatx4 acc[8][8];
  gemm_mainloop16<F16>(c, acc);

  // lane l of block (i, j) holds column l % 16 and rows 4·(l/16) + v
  const int lane = threadIdx.x & 63;
  const int wm = c.wave >> 1, wn = c.wave & 1;
  const int64_t row0 = m0 + wm * 128 + 4 * (lane >> 4);
  const int64_t col0 = n0 + wn * 128 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t col = col0 + j * 16;
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = row0 + i * 16 + v;
        if (row < M) Y[row * N + col] = to16<F16>(acc[i][j][v]);
      }
    }
}

// ---------------------------------------------------------------------------
// prefill, dequantising on the fly: X tiles through the LDS-DMA ring, the B
// tile formed from the packed layer in registers
// ---------------------------------------------------------------------------
//
// The same 256x256 tiles and 16x16x32 main loop as the GEMM above (the
// 64-wide, 2-stage ring of gemm_core.h); only the B operand reaches LDS from
// registers instead of by DMA. Lane (j, kc) = (tid % 32, tid / 32) owns word
// column j of the output tile (outputs n0 + 8j .. + 7) and k rows 8kc .. 8kc + 7
// of each 64-wide k-tile: 8 qweight words, its group's zero-point word and the
// 8 fp16 scales (32 lanes read 128 consecutive bytes of a qweight row). Region
// kt (whose MFMAs read k-tile kt) loads the packed k-tile kt + 2 into the slot
// k-tile kt used and forms the operand of k-tile kt + 1, as the DMA of X's
// k-tile kt + 1 fills the same ring stage. Each output row's 8 k values are
// one 16-byte LDS store. An LDS write serves 8 lanes at a time, which must
// hit 8 different 16-byte bank groups (chunk slots modulo 8); lane j takes
// its rows in the order i + 2t (mod 8), t = (j / 2) % 4, which puts the 8
// lanes j = 8b .. 8b + 7 on 8 distinct slots of the swizzled layout. That is
// a rotation of the words by whole bytes (so the nibble classes below keep
// their parity) and of the scales by whole words.
//
// Ŵ = (q − z)·scale as the dequantisation pass rounds it, with one
// v_fma_mix_f32 per value: the code enters as an fp16 number B + q whose low
// mantissa bits are the nibble (B = 1024 for a nibble at bits 0..3 of a
// 16-bit half, 0x6400 | q; B = 64 for one at bits 4..7, 0x5400 | q << 4),
// made by one and-or of the word (or of the word shifted right by 8); the
// scale enters as its fp16 half; the addend is −(B + z)·scale, formed the
// same way from the zero-point word. (B + q)·scale and (B + z)·scale have at
// most 22 significant bits, so the fused result is (q − z)·scale rounded once
// to float32, the value the dequantisation pass forms, and the operand equals
// that pass's bit for bit.

// Tile order of this kernel: from 32 token tiles on the shared XCD-grouped
// order; below that, column tile by column tile with the token tile fastest,
// so consecutive ids (one per XCD in turn) spread each column tile's packed
// words over the XCDs. The grouped order for 4-16 token tiles suits the
// two-pass GEMM, whose B tiles are as large as its A tiles; here B is a
// quarter of the bytes and the grouped order measured slower.
__device__ __forceinline__ bool q_tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  if (tiles_m >= 32) return tile_of(bid, tiles_m, tiles_n, tm, tn);
  tm = bid % tiles_m;
  tn = bid / tiles_m;
  return tn < tiles_n;
}

inline int64_t q_gemm_blocks(int tiles_m, int tiles_n) {
  return tiles_m >= 32 ? gemm_blocks(tiles_m, tiles_n) : int64_t(tiles_m) * tiles_n;
}

struct Q16Slot {
  uint32_t w[8];   // qweight words of k rows 8kc .. 8kc + 7
  uint32_t z;      // zero-point word
  uint4 s;         // 8 fp16 scales
};

struct Q16Ctx {
  __amdgpu_buffer_rsrc_t rsQ, rsZ, rsS;
  // Vector offsets (bytes, bit 31 set for a lane whose word column is past
  // N, so its loads read zero): the lane's qweight word at k row 8kc of
  // k-tile 0, and its zero-point word and scales in the group that k row
  // 64·kt + 8kc falls in, less the part common to the wave (g0(kt) group rows)
  uint32_t qoff, zoff, soff;
  uint32_t qrow, ktq, zrow, srow;   // bytes per k row, per k-tile, per group row (two)
  int kt_last;               // the last k-tile
  int gshift;                // log2 of the group size
  uint32_t rot;              // 8t: the words' rotation in bits
  bool t2, t1;               // t & 2, t & 1: the scale words' rotation
  int lds[8];                // LDS byte offset within a stage of the lane's row i
  uint32_t mag[2];           // 0x64006400 and 0x54005400, kept in vector registers
};

constexpr uint32_t kQOob = 0x80000000u;  // past every buffer: loads read zero

// The wave's first group row of k-tile kt: k rows 64·kt .. + 63 hold groups
// 2kt and 2kt + 1 at group size 32 (the lane's share is in q.zoff, q.soff),
// group kt at 64 and kt / 2 at 128.
__device__ __forceinline__ uint32_t q16_group0(const Q16Ctx& q, int kt) {
  return q.gshift == 5 ? uint32_t(2 * kt) : uint32_t(kt) >> (q.gshift - 6);
}

// Packed k-tile kt of this lane. The k-tile's and the group's steps are
// common to the wave, so they go in the scalar offsets; k-tiles past the
// last one (loaded ahead, never used) read the last one again.
__device__ __forceinline__ void q16_load(const Q16Ctx& q, int kt, Q16Slot& sl) {
  const int k = kt < q.kt_last ? kt : q.kt_last;
  const uint32_t sq = uint32_t(k) * q.ktq, g = q16_group0(q, k);
#pragma unroll
  for (int r = 0; r < 8; ++r)
    sl.w[r] = __builtin_amdgcn_raw_buffer_load_b32(q.rsQ, q.qoff, int(sq + r * q.qrow), 0);
  sl.z = __builtin_amdgcn_raw_buffer_load_b32(q.rsZ, q.zoff, int(g * q.zrow), 0);
  const auto sv = __builtin_amdgcn_raw_buffer_load_b128(q.rsS, q.soff, int(g * q.srow), 0);
  sl.s = make_uint4(sv[0], sv[1], sv[2], sv[3]);
}

// fp16 numbers B + nibble in both 16-bit halves of a word (see above): NIB = 0
// takes the nibbles at bits 0..3 of each half (B = 1024), NIB = 1 those at
// bits 4..7 (B = 64). One v_and_or_b32: the mask comes from a scalar
// register and the exponent bits from a vector register that q.mag holds
// (two literals cannot share one instruction here).
template <int NIB>
__device__ __forceinline__ uint32_t magic16(const Q16Ctx& q, uint32_t x) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3"
      : "=v"(r)
      : "v"(x), "s"(NIB == 0 ? 0x000F000Fu : 0x00F000F0u), "v"(q.mag[NIB]));
  return r;
}

// float32 a·b + c with a and b the fp16 halves HA / HB of their words (NA
// negates a): one v_fma_mix_f32, whose fp16 inputs are exact in float32
template <int HA, int HB, bool NA>
__device__ __forceinline__ float fma_mix16(uint32_t a, uint32_t b, float c) {
  float r;
  if constexpr (NA) {
    if constexpr (HA == 0 && HB == 0)
      asm("v_fma_mix_f32 %0, -%1, %2, %3 op_sel_hi:[1,1,0]" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    else if constexpr (HA == 0)
      asm("v_fma_mix_f32 %0, -%1, %2, %3 op_sel:[0,1,0] op_sel_hi:[1,1,0]"
          : "=v"(r) : "v"(a), "v"(b), "v"(c));
    else if constexpr (HB == 0)
      asm("v_fma_mix_f32 %0, -%1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,1,0]"
          : "=v"(r) : "v"(a), "v"(b), "v"(c));
    else
      asm("v_fma_mix_f32 %0, -%1, %2, %3 op_sel:[1,1,0] op_sel_hi:[1,1,0]"
          : "=v"(r) : "v"(a), "v"(b), "v"(c));
  } else {
    if constexpr (HA == 0 && HB == 0)
      asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,1,0]" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    else if constexpr (HA == 0)
      asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[1,1,0]"
          : "=v"(r) : "v"(a), "v"(b), "v"(c));
    else if constexpr (HB == 0)
      asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,1,0]"
          : "=v"(r) : "v"(a), "v"(b), "v"(c));
    else
      asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,1,0] op_sel_hi:[1,1,0]"
          : "=v"(r) : "v"(a), "v"(b), "v"(c));
  }
  return r;
}

// two float32 values rounded to nearest even into one packed 16-bit pair
// (low half first), the conversion the dequantisation pass applies to each
template <bool F16>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  uint32_t r;
  if constexpr (F16) asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  else asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Forming one k-tile's operand: the lane's row i (output row 8j + (i + 2t)
// % 8) takes nibble i of each rotated word (bits 4i .. 4i + 3), so nibble
// class c = i % 4 (the and-or on the rotated word for c < 2, on it shifted
// right by 8 for c >= 2; low nibbles for even c) holds rows c and c + 4 in
// its two halves. Operations, at most two VALU instructions each (what a
// 16x16x32 MFMA hides), none reading what the one just before it wrote:
//  * C a: X's DMA copy a of the next k-tile;
//  * RA h, RB h: the scale words rotated by 2 words, then by 1 (h = which
//    pair of the four);
//  * ZR, ZA, ZT, ZB: the zero-point word rotated, its classes 0 and 1, its
//    shift, classes 2 and 3;
//  * N c: −(B + z)·scale of rows c and c + 4;
//  * X p: words 2p and 2p + 1 rotated;  T p: those shifted right by 8;
//  * M c p: class c of words 2p and 2p + 1;
//  * V c p h: the values of row c (h = 0) or c + 4 (h = 1) at k rows 2p and
//    2p + 1;
//  * P c p: those values packed, for both rows;
//  * D c: the 16-byte LDS stores of rows c and c + 4.
struct Q16Work {
  uint32_t x[8];     // rotated words
  uint32_t a[4], sw[4], zx;   // scale words rotated by 2 words, then by t; rotated zero word
  uint32_t t[8];     // rotated words shifted right by 8
  uint32_t m[8];     // the current class of each word
  uint32_t zm[4], zt;
  float nzs[8];
  float v[4];        // the values of pair p: row c at 2p, 2p + 1; row c + 4 at 2p, 2p + 1
  uint32_t h[2][4];  // packed k pairs of rows c and c + 4
};

constexpr int kQ16Copy = 1, kQ16RA = 2, kQ16RB = 3, kQ16ZR = 4, kQ16ZA = 5, kQ16ZT = 6,
              kQ16ZB = 7, kQ16N = 8, kQ16X = 9, kQ16T = 10, kQ16M = 11, kQ16V = 12,
              kQ16P = 13;
constexpr int q16_code(int kind, int a = 0, int b = 0) { return kind * 100 + a * 10 + b; }

// The schedule of a region's 128 MFMA slots: slot s runs q16_op_at(s) (0 =
// none) after MFMA s, and the stores q16_store_at(s) (−1 = none). Every
// operation is at least two slots after those it reads.
//  slots 0..31: copies, then X 0..3, then T 0..3 in the even slots; RA, RB,
//  the zero-point word and N 0..3 in the odd;
//  slots 32..97: the classes in order 0..3, 16 slots each, pair p of class
//  c taking slots 4p .. 4p + 3 of it for M c p, P c (p − 1) (the previous
//  class's last pack at p = 0), V c p 0 and V c p 1; class c's stores go
//  two slots after its last pack.
constexpr int kQ16Classes = 32;   // first slot of class 0; class c starts 16c later
constexpr int q16_op_at(int s) {
  if (s < 32) {
    if (s % 2 == 0) {
      const int e = s / 2;
      return e < 8 ? q16_code(kQ16Copy, e) : e < 12 ? q16_code(kQ16X, e - 8)
                                                     : q16_code(kQ16T, e - 12);
    }
    constexpr int odd[16] = {q16_code(kQ16RA, 0), q16_code(kQ16RA, 1), q16_code(kQ16ZR),
                             q16_code(kQ16RB, 0), q16_code(kQ16RB, 1), q16_code(kQ16ZA),
                             q16_code(kQ16ZT),    q16_code(kQ16ZB),    q16_code(kQ16N, 0),
                             q16_code(kQ16N, 1),  q16_code(kQ16N, 2),  q16_code(kQ16N, 3),
                             0, 0, 0, 0};
    return odd[s / 2];
  }
  const int d = s - kQ16Classes;
  if (d == 65) return q16_code(kQ16P, 3, 3);
  if (d < 64) {
    const int c = d / 16, p = (d % 16) / 4, e = d % 4;
    if (e == 0) return q16_code(kQ16M, c, p);
    if (e == 1) return p > 0 ? q16_code(kQ16P, c, p - 1) : c > 0 ? q16_code(kQ16P, c - 1, 3) : 0;
    return q16_code(kQ16V, c, 2 * p + (e - 2));
  }
  return 0;
}
constexpr int q16_store_at(int s) {
  const int d = s - kQ16Classes - 16 - 3;   // two slots after class c's last pack
  return d >= 0 && d <= 48 && d % 16 == 0 ? d / 16 : -1;
}

template <bool F16, int S, int OP, bool COPY = true>
__device__ __forceinline__ void q16_op(const GemmCtx64& c, const Q16Ctx& q, const Q16Slot& sl,
                                       Q16Work& w, int kt) {
  constexpr int kind = OP / 100, A = (OP / 10) % 10, B = OP % 10;
  if constexpr (kind == kQ16Copy) {
    if constexpr (COPY) copy64<S>(c, kt + 1, A);
  } else if constexpr (kind == kQ16RA) {
    // scale word k of the result is word (k + t) % 4 of the slot's (selects,
    // not branches: the loop body stays one block)
    if constexpr (A == 0) {
      w.a[0] = q.t2 ? sl.s.z : sl.s.x;
      w.a[1] = q.t2 ? sl.s.w : sl.s.y;
    } else {
      w.a[2] = q.t2 ? sl.s.x : sl.s.z;
      w.a[3] = q.t2 ? sl.s.y : sl.s.w;
    }
  } else if constexpr (kind == kQ16RB) {
    w.sw[2 * A] = q.t1 ? w.a[2 * A + 1] : w.a[2 * A];
    w.sw[2 * A + 1] = q.t1 ? w.a[(2 * A + 2) % 4] : w.a[2 * A + 1];
  } else if constexpr (kind == kQ16ZR) {
    w.zx = __builtin_amdgcn_alignbit(sl.z, sl.z, q.rot);
  } else if constexpr (kind == kQ16ZA) {
    w.zm[0] = magic16<0>(q, w.zx);
    w.zm[1] = magic16<1>(q, w.zx);
  } else if constexpr (kind == kQ16ZT) {
    w.zt = w.zx >> 8;
  } else if constexpr (kind == kQ16ZB) {
    w.zm[2] = magic16<0>(q, w.zt);
    w.zm[3] = magic16<1>(q, w.zt);
  } else if constexpr (kind == kQ16N) {
    // rows A and A + 4: scales in rotated words A / 2 and 2 + A / 2, half A % 2
    w.nzs[A] = fma_mix16<0, A % 2, true>(w.zm[A], w.sw[A / 2], 0.0f);
    w.nzs[A + 4] = fma_mix16<1, A % 2, true>(w.zm[A], w.sw[2 + A / 2], 0.0f);
  } else if constexpr (kind == kQ16X) {
    w.x[2 * A] = __builtin_amdgcn_alignbit(sl.w[2 * A], sl.w[2 * A], q.rot);
    w.x[2 * A + 1] = __builtin_amdgcn_alignbit(sl.w[2 * A + 1], sl.w[2 * A + 1], q.rot);
  } else if constexpr (kind == kQ16T) {
    w.t[2 * A] = w.x[2 * A] >> 8;
    w.t[2 * A + 1] = w.x[2 * A + 1] >> 8;
  } else if constexpr (kind == kQ16M) {
    const uint32_t x0 = A < 2 ? w.x[2 * B] : w.t[2 * B];
    const uint32_t x1 = A < 2 ? w.x[2 * B + 1] : w.t[2 * B + 1];
    w.m[2 * B] = magic16<A % 2>(q, x0);
    w.m[2 * B + 1] = magic16<A % 2>(q, x1);
  } else if constexpr (kind == kQ16V) {
    constexpr int p = B / 2, h = B % 2;   // row A + 4h, k rows 2p and 2p + 1
    const uint32_t s = w.sw[2 * h + A / 2];
    w.v[2 * h] = fma_mix16<h, A % 2, false>(w.m[2 * p], s, w.nzs[A + 4 * h]);
    w.v[2 * h + 1] = fma_mix16<h, A % 2, false>(w.m[2 * p + 1], s, w.nzs[A + 4 * h]);
  } else if constexpr (kind == kQ16P) {
    w.h[0][B] = pack16<F16>(w.v[0], w.v[1]);
    w.h[1][B] = pack16<F16>(w.v[2], w.v[3]);
  }
}

// the 16-byte stores of rows c and c + 4 into stage S
template <int S, int C>
__device__ __forceinline__ void q16_store(const Q16Ctx& q, const Q16Work& w) {
  char* base = reinterpret_cast<char*>(stage64_b<S>());
  *reinterpret_cast<uint4*>(base + q.lds[C]) =
      make_uint4(w.h[0][0], w.h[0][1], w.h[0][2], w.h[0][3]);
  *reinterpret_cast<uint4*>(base + q.lds[C + 4]) =
      make_uint4(w.h[1][0], w.h[1][1], w.h[1][2], w.h[1][3]);
}

// All of one slot's operand into stage S (the prologue; copies left out).
template <bool F16, int S, int... Ss>
__device__ __forceinline__ void q16_form_seq(const GemmCtx64& c, const Q16Ctx& q,
                                             const Q16Slot& sl, Q16Work& w,
                                             std::integer_sequence<int, Ss...>) {
  (([&] {
     q16_op<F16, S, q16_op_at(Ss), false>(c, q, sl, w, 0);
     if constexpr (q16_store_at(Ss) >= 0) q16_store<S, q16_store_at(Ss)>(q, w);
   }()),
   ...);
}
template <bool F16, int S>
__device__ __forceinline__ void q16_form_all(const GemmCtx64& c, const Q16Ctx& q,
                                             const Q16Slot& sl) {
  Q16Work w;
  q16_form_seq<F16, S>(c, q, sl, w, std::make_integer_sequence<int, 128>{});
}

// MFMA m of region kt (stage S = kt % 2) and what follows it. MFMAs 0..63
// finish the previous k-step (fragments f1; none in the first region) and
// read k-step 0's fragments f0 after every fourth; MFMAs 64..127 run k-step
// 0 and read k-step 1's into f1. Then slot m's operation for the operand of
// k-tile kt + 1 (into stage S ^ 1), pinned there.
template <bool F16, int S, bool PREV, int M, class V>
__device__ __forceinline__ void q16_slot(const GemmCtx64& c, const Q16Ctx& q,
                                         const int (&rdA)[2], const int (&rdB)[2], int kt,
                                         floatx4 (&acc)[8][8], V (&f0a)[8], V (&f0b)[8],
                                         V (&f1a)[8], V (&f1b)[8], const Q16Slot& sl,
                                         Q16Work& w) {
  constexpr int u = (M % 64) / 4, t = M % 4, i = u >> 1, j = (u & 1) * 4 + t;
  if constexpr (M < 64) {
    if constexpr (PREV) mfma16(acc[i][j], f1a[i], f1b[j]);
    if constexpr (t == 0) frag16<S>(rdA[0], rdB[0], u, f0a, f0b);
  } else {
    mfma16_acc<!PREV>(acc[i][j], f0a[i], f0b[j]);
    if constexpr (t == 0) frag16<S>(rdA[1], rdB[1], u, f1a, f1b);
  }
  constexpr int op = q16_op_at(M), st = q16_store_at(M);
  if constexpr (op != 0 || st >= 0) {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (st >= 0) q16_store<S ^ 1, st>(q, w);
    if constexpr (op != 0) q16_op<F16, S ^ 1, op>(c, q, sl, w, kt);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <bool F16, int S, bool PREV, class V, int... Ms>
__device__ __forceinline__ void q16_slots(const GemmCtx64& c, const Q16Ctx& q,
                                          const int (&rdA)[2], const int (&rdB)[2], int kt,
                                          floatx4 (&acc)[8][8], V (&f0a)[8], V (&f0b)[8],
                                          V (&f1a)[8], V (&f1b)[8], const Q16Slot& sl,
                                          Q16Work& w, std::integer_sequence<int, Ms...>) {
  (q16_slot<F16, S, PREV, Ms>(c, q, rdA, rdB, kt, acc, f0a, f0b, f1a, f1b, sl, w), ...);
}

// Region kt (stage S = kt % 2): the packed loads of k-tile kt + 2 go out
// first, into the slot k-tile kt was formed from; the 128 MFMA slots follow;
// the region ends, as in gemm_core.h, with one wait and one barrier.
template <bool F16, int S, bool PREV, class V>
__device__ __forceinline__ void region16q(const GemmCtx64& c, const Q16Ctx& q,
                                          const int (&rdA)[2], const int (&rdB)[2], int kt,
                                          floatx4 (&acc)[8][8], V (&f0a)[8], V (&f0b)[8],
                                          V (&f1a)[8], V (&f1b)[8], Q16Slot (&slot)[2]) {
  Q16Work w;
  q16_load(q, kt + 2, slot[S]);
  __builtin_amdgcn_sched_barrier(0);
  q16_slots<F16, S, PREV>(c, q, rdA, rdB, kt, acc, f0a, f0b, f1a, f1b, slot[S ^ 1], w,
                          std::make_integer_sequence<int, 128>{});
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  region_barrier();
}

template <bool F16>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void w4a16_gemm_q_kernel(const uint16_t* __restrict__ X, const int32_t* __restrict__ qweight,
                         const int32_t* __restrict__ qzeros, const uint16_t* __restrict__ scales,
                         int64_t M, int64_t N, int64_t K, int gshift, int tiles_m, int tiles_n,
                         uint16_t* __restrict__ Y) {
  typedef typename Operand<F16>::type V;
  int tm, tn;
  if (!q_tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;
  const int64_t rows_a = M - m0 < BM ? M - m0 : BM;
  const int tid = threadIdx.x;
  // X through the ring (B's half of the context is unused: B is formed here)
  GemmCtx64 c;
  gemm_setup64(c, X + m0 * K, rows_a, X + m0 * K, rows_a, K);
  Q16Ctx q;
  const int64_t N8 = N / 8, G = int64_t(1) << gshift;
  q.rsQ = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(qweight), 0,
                                            int(K * N8 * 4), 0x00020000);
  q.rsZ = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(qzeros), 0,
                                            int(K / G * N8 * 4), 0x00020000);
  q.rsS = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales), 0,
                                            int(K / G * N * 2), 0x00020000);
  const int j = tid & 31, kc = tid >> 5;
  const int64_t col = n0 / 8 + j;  // word column
  const uint32_t oobm = col < N8 ? 0u : kQOob;
  q.qrow = uint32_t(N8 * 4);
  q.ktq = q.qrow * 64;
  q.zrow = uint32_t(N8 * 4);
  q.srow = uint32_t(N * 2);
  q.kt_last = int(K / 64) - 1;
  q.gshift = gshift;
  // at group size 32 the lane's k rows 8kc .. 8kc + 7 sit in the k-tile's
  // second group for kc >= 4
  const uint32_t gl = gshift == 5 ? uint32_t(kc >> 2) : 0u;
  q.qoff = uint32_t((int64_t(8 * kc) * N8 + col) * 4) | oobm;
  q.zoff = (uint32_t(col * 4) + gl * q.zrow) | oobm;
  q.soff = (uint32_t(col * 16) + gl * q.srow) | oobm;
  const int t = (j >> 1) & 3;
  q.rot = uint32_t(8 * t);
  q.t2 = t & 2;
  q.t1 = t & 1;
  // row m = (i + 2t) % 8 of the lane's 8 sits at swz64(8j + m, kc)·16
#pragma unroll
  for (int i = 0; i < 8; ++i) q.lds[i] = swz64(8 * j + ((i + 2 * t) & 7), kc) * 16;
  // opaque to the compiler, so it keeps them in registers instead of
  // re-materialising them at every use
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(q.mag[0]));
  asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(q.mag[1]));

  int rdA[2], rdB[2];
  frag_offsets16(c, rdA, rdB);
  floatx4 acc[8][8];
  // prologue: k-tile 0 of X and of the operand in stage 0; packed k-tile 1
  // in slot 1, which region 0 forms from
  Q16Slot slot[2];
  q16_load(q, 0, slot[0]);
  q16_load(q, 1, slot[1]);
  dma64_a<0>(c, 0);
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  q16_form_all<F16, 0>(c, q, slot[0]);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  region_barrier();
  V f0a[8], f0b[8], f1a[8], f1b[8];
  region16q<F16, 0, false>(c, q, rdA, rdB, 0, acc, f0a, f0b, f1a, f1b, slot);
  int kt = 1;
  for (; kt + 1 < c.KT; kt += 2) {
    region16q<F16, 1, true>(c, q, rdA, rdB, kt, acc, f0a, f0b, f1a, f1b, slot);
    region16q<F16, 0, true>(c, q, rdA, rdB, kt + 1, acc, f0a, f0b, f1a, f1b, slot);
  }
  if (kt < c.KT) region16q<F16, 1, true>(c, q, rdA, rdB, kt, acc, f0a, f0b, f1a, f1b, slot);
  mfma_8x8(acc, f1a, f1b);
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) asm volatile("" : "+a"(acc[i][jj]));

  // lane l of block (i, j) holds column l % 16 and rows 4·(l/16) + v
  const int lane = tid & 63;
  const int wm = c.wave >> 1, wn = c.wave & 1;
  const int64_t row0 = m0 + wm * 128 + 4 * (lane >> 4);
  const int64_t col0 = n0 + wn * 128 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int64_t cn = col0 + jj * 16;
      if (cn >= N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = row0 + i * 16 + v;
        if (row < M) Y[row * N + cn] = to16<F16>(acc[i][jj][v]);
      }
    }
}

// ---------------------------------------------------------------------------
// decode: fused GEMV
// ---------------------------------------------------------------------------

constexpr int kGemvCols = 64;     // word columns per workgroup (512 outputs)
constexpr int kGemvWaves = 4;     // k runs per workgroup

// Workgroup (cb, kc): word columns cb·64 .. cb·64+63, k rows kc·(4·kpw) ..;
// wave w takes rows kc·4·kpw + w·kpw .. + kpw - 1. Lane = word column.
// TT >= T is the register tile of token rows; rows T..TT-1 are zeros that
// are neither read from X nor written.
//
// Per qweight word (8 output channels at one k): the nibbles are split into
// bytes (w & 0x0F0F0F0F and (w >> 4) & 0x0F0F0F0F) and converted with the
// byte-to-float instructions; ŵ = fma(q, scale, -z·scale) is exact (every
// term is an integer of at most 4 bits times an fp16 value); then one FMA per
// token row. Activations sit in LDS as [k][TT] so four token rows come in
// one 16-byte read.
template <bool F16, int TT>
__global__ __launch_bounds__(256) void w4a16_gemv_kernel(
    const uint16_t* __restrict__ X, int64_t T, int64_t N, int64_t K,
    const int32_t* __restrict__ qweight, const int32_t* __restrict__ qzeros,
    const uint16_t* __restrict__ scales, int group, int kpw, float* __restrict__ partial) {
  constexpr int TR = TT < 4 ? TT : 4;            // token rows per cross-wave reduction pass
  __shared__ float xs[kGemvWaves * 128][TT];
  __shared__ float red[kGemvWaves - 1][TR][kGemvCols * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t N8 = N / 8;
  const int64_t j = int64_t(blockIdx.x) * kGemvCols + lane;
  const int64_t kchunk = int64_t(kGemvWaves) * kpw;
  const int64_t kbase = int64_t(blockIdx.y) * kchunk;
  // stage this chunk's activations as float32 (rows past T as zeros)
  for (int e = threadIdx.x; e < TT * kchunk; e += 256) {
    const int t = e / int(kchunk), kk = e % int(kchunk);
    xs[kk][t] = t < T ? from16<F16>(X[t * K + kbase + kk]) : 0.f;
  }
  __syncthreads();

  float acc[TT][8];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[t][r] = 0.f;

  if (j < N8) {
    const int64_t k0 = kbase + int64_t(wave) * kpw;
    float sc[8], zs[8];
    int64_t g_cur = -1;
    for (int kk = 0; kk < kpw; kk += 8) {
      const int64_t k = k0 + kk;
      if (k / group != g_cur) {
        g_cur = k / group;
        float zf[8];
        group_params(qzeros, scales, N, g_cur, j, sc, zf);
#pragma unroll
        for (int r = 0; r < 8; ++r) zs[r] = -(zf[r] * sc[r]);
      }
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = uint32_t(qweight[(k + i) * N8 + j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t ev = w[i] & 0x0F0F0F0Fu, od = (w[i] >> 4) & 0x0F0F0F0Fu;
        float q[8];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          q[2 * b] = float((ev >> (8 * b)) & 0xFFu);
          q[2 * b + 1] = float((od >> (8 * b)) & 0xFFu);
        }
        float xv[TT];
        const int xk = wave * kpw + kk + i;
#pragma unroll
        for (int t = 0; t < TT; ++t) xv[t] = xs[xk][t];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float wv = __builtin_fmaf(q[r], sc[r], zs[r]);
#pragma unroll
          for (int t = 0; t < TT; ++t) acc[t][r] = __builtin_fmaf(xv[t], wv, acc[t][r]);
        }
      }
    }
  }
  // waves 1..3 hand their sums to wave 0, TR token rows at a time
#pragma unroll
  for (int t0 = 0; t0 < TT; t0 += TR) {
    if (t0 > 0) __syncthreads();
    if (wave > 0) {
#pragma unroll
      for (int t = 0; t < TR; ++t)
#pragma unroll
        for (int r = 0; r < 8; ++r) red[wave - 1][t][lane * 8 + r] = acc[t0 + t][r];
    }
    __syncthreads();
    if (wave == 0 && j < N8) {
#pragma unroll
      for (int t = 0; t < TR; ++t) {
        if (t0 + t >= T) break;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float s = ((acc[t0 + t][r] + red[0][t][lane * 8 + r]) + red[1][t][lane * 8 + r]) +
                          red[2][t][lane * 8 + r];
          partial[(int64_t(blockIdx.y) * T + t0 + t) * N + 8 * j + r] = s;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// decode on the matrix cores: exact integer codes against the activations
// ---------------------------------------------------------------------------
//
// Per group g of k rows, Σ_k x·ŵ = scale·Σ_k x·(q − z). The codes enter the
// MFMA as B = 1 + q/16, built from the bits: q goes into the top four
// mantissa bits of a 16-bit float of exponent 0 (bf16 0x3F80 | q << 3, fp16
// 0x3C00 | q << 6). Every x·B has at most 16 significant bits, so the
// v_mfma_f32_16x16x32 products are exact and P'[t][n] = Σ_k x[t][k]·B[k][n]
// is an ordinary float32 sum. One more MFMA against a column of ones gives
// S[t] = Σ_k x[t][k], and Σ_k x·(q − z) = 16·P' − (16 + z)·S. After each
// 32-row k-block a lane adds scale·(P' − ((16 + z)/16)·S) to its float32
// totals (scaled by 16 once at the end). Token rows past T read row 0 and
// are never stored.
//
// Operand layout (16x16x32): lane l holds 8 consecutive k (k = 8·(l/16) + e)
// of row l % 16 of A and of column l % 16 of B, and receives D[4·(l/16) + v]
// [l % 16] for v = 0..3. The contraction only needs A and B to agree on which
// k each (lane group, element) holds, so a lane loads k rows 8·(l/16) + e of
// its qweight words and each nibble position r of a word feeds its own MFMA:
// MFMA (c, r) covers output channels 8·(wc + c) + r over the 16 lanes' word
// columns wc. A is read straight from X (16 bytes per lane and k-block).
//
// Workgroup (cb, kc): 4 waves, 256 outputs (a lane owns 16: two adjacent
// 4-bit word columns, one 8-byte load per k row, or half of a 3-bit group of
// 32), k rows kc·4·kpw ..;
// wave w takes kpw of them (a multiple of 32), and the waves' totals meet in
// LDS in a fixed order before one float32 partial per (kc, t, n) is stored.
constexpr int kMgWaves = 4;
constexpr int kMgCols = 32;       // word columns per workgroup
constexpr int kMgMfma = 16;       // (c, r): 2 word columns x 8 nibbles per lane

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma16(bf16x8_t a, bf16x8_t b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(f16x8_t a, f16x8_t b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// B = 1 + q/16 for nibble r of two qweight words (two consecutive k rows),
// packed as a pair of 16-bit floats (lo word in the low half). v_perm puts
// byte r/2 of each word at bits 0-7 and 16-23; one shift moves the nibble to
// the top four mantissa bits and one and-or masks it and sets the exponent.
// The other bytes perm and the shift bring along fall outside the mask.
template <bool F16, int R>
__device__ __forceinline__ uint32_t code_pair(uint32_t w_lo, uint32_t w_hi) {
  constexpr uint32_t b = R >> 1;
  const uint32_t x = __builtin_amdgcn_perm(w_hi, w_lo, 0x0C000C00u | ((4u + b) << 16) | b);
  // nibble at bits 0-3 (R even) or 4-7 (R odd) of each half -> mantissa top
  constexpr int kTop = F16 ? 6 : 3;          // lowest bit of the top 4 mantissa bits
  constexpr int kShift = kTop - 4 * (R & 1);
  const uint32_t y = kShift >= 0 ? (x << kShift) : (x >> -kShift);
  constexpr uint32_t kMask = F16 ? 0x03C003C0u : 0x00780078u;
  constexpr uint32_t kOne = F16 ? 0x3C003C00u : 0x3F803F80u;
  return (y & kMask) | kOne;
}

// The 3-bit layout keeps a 32-row group's codes in 3 words; the two lanes
// that share a group each load 2 of them (words 0-1 or 1-2) and funnel-shift
// their 64 bits right by 0 or 16, so that both hold their 16 codes at bits
// 3r .. 3r+2 of a 48-bit value (lo, hi): codes 0-9 in lo, 11-15 in hi, and
// code 10 across the two. B = 1 + q/16 for code R of two consecutive k rows,
// as code_pair: v_perm takes a 2-byte window holding the code from each
// row's word, one shift puts it at the mantissa bits of q/16 and one and-or
// masks it and sets the exponent (the bits the shift carries across the
// halves fall outside the mask).
template <bool F16, int R>
__device__ __forceinline__ uint32_t code3_pair(uint32_t lo_a, uint32_t hi_a, uint32_t lo_b,
                                               uint32_t hi_b, uint32_t one) {
  constexpr int kLow = F16 ? 6 : 3;          // lowest mantissa bit of q/16
  constexpr int b = R < 10 ? 3 * R : R > 10 ? 3 * R - 32 : 0;
  uint32_t wa, wb;
  if constexpr (R < 10) {
    wa = lo_a;
    wb = lo_b;
  } else if constexpr (R > 10) {
    wa = hi_a;
    wb = hi_b;
  } else {
    wa = __builtin_amdgcn_alignbit(hi_a, lo_a, 30);
    wb = __builtin_amdgcn_alignbit(hi_b, lo_b, 30);
  }
  constexpr uint32_t B0 = (b >> 3) < 2 ? uint32_t(b >> 3) : 2u;
  constexpr int kShift = b - 8 * int(B0) - kLow;
  const uint32_t x =
      __builtin_amdgcn_perm(wb, wa, B0 | ((B0 + 1u) << 8) | ((B0 + 4u) << 16) | ((B0 + 5u) << 24));
  const uint32_t y = kShift >= 0 ? (x >> kShift) : (x << -kShift);
  constexpr uint32_t kMask = (7u << kLow) | (7u << (16 + kLow));
  return (y & kMask) | one;
}

// Code r of a lane's aligned 48-bit value (lo, hi), as an integer.
template <int R>
__device__ __forceinline__ uint32_t code3_at(uint32_t lo, uint32_t hi) {
  if constexpr (R < 10) return (lo >> (3 * R)) & 7u;
  else if constexpr (R > 10) return (hi >> (3 * R - 32)) & 7u;
  else return __builtin_amdgcn_alignbit(hi, lo, 30) & 7u;
}

// Registers of one wave: totals per MFMA (c, r); four k-block slots (codes,
// activations, and the group parameters when the block opens a group: raw
// fp16 scale pairs and packed zero points), of which three are live at a
// time (two blocks are prefetched ahead); and the open group's scales and
// decoded zero points.
constexpr int kMgSlots = 4;

template <bool F16>
struct MgState {
  floatx4 tot[kMgMfma];
  floatx4 pacc[kMgMfma], sacc;  // the open group's MFMA sums P' and S
  uint2 w[kMgSlots][8];
  uint4 a[kMgSlots];
  uint4 ps0[kMgSlots], ps1[kMgSlots];
  uint2 pz[kMgSlots];
  uint4 s0, s1;
  float zf[kMgMfma];
};

// Block j (0..3) of a 128-row super-block starting at kb, for groups of G
// rows (a 128-row super-block holds whole groups, so j's place in its group
// is known here): at a group's first block take its parameters from the
// block's slot; prefetch block j + 2 into slot (j + 2) % 4 (with its group's
// parameters if it opens one); then S = Σ x and, per (c, r), P' = Σ x·B
// from zero, folded at once: tot += scale·(P' − ((16 + z)/16)·S). That is
// scale·(16·P' − (16 + z)·S) / 16 with the same rounding; the factor 16 is
// applied once at the end.
template <bool F16, int BITS, int G, int TV, int J, class LoadData, class LoadPar>
__device__ __forceinline__ void mg_block(MgState<F16>& st, int kb, const LoadData& load_data,
                                         const LoadPar& load_par, uint32_t one) {
  typedef typename Operand<F16>::type V;
  constexpr int BPG = G / 32;
  constexpr bool kFirst = J % BPG == 0;
  constexpr bool kAheadOpens = (J + 2) % BPG == 0;
  constexpr int B = J & 3, BA = (J + 2) & 3;
  // 3 bits: this lane's funnel shift (0 or 16, by the parity of its group
  // half)
  const uint32_t sh3 = (threadIdx.x & 1u) << 4;
  if constexpr (kFirst) {
    st.s0 = st.ps0[B];
    st.s1 = st.ps1[B];
    if constexpr (BITS == 4) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        st.zf[r] = float(16u + ((st.pz[B].x >> (4 * r)) & 0xFu)) * 0.0625f;
        st.zf[8 + r] = float(16u + ((st.pz[B].y >> (4 * r)) & 0xFu)) * 0.0625f;
      }
    } else {
      const uint32_t zl = __builtin_amdgcn_alignbit(st.pz[B].y, st.pz[B].x, sh3);
      const uint32_t zh = st.pz[B].y >> sh3;
#define AWQ_MG_Z3(R) st.zf[R] = float(16u + code3_at<R>(zl, zh)) * 0.0625f;
      AWQ_MG_Z3(0) AWQ_MG_Z3(1) AWQ_MG_Z3(2) AWQ_MG_Z3(3) AWQ_MG_Z3(4) AWQ_MG_Z3(5)
      AWQ_MG_Z3(6) AWQ_MG_Z3(7) AWQ_MG_Z3(8) AWQ_MG_Z3(9) AWQ_MG_Z3(10) AWQ_MG_Z3(11)
      AWQ_MG_Z3(12) AWQ_MG_Z3(13) AWQ_MG_Z3(14) AWQ_MG_Z3(15)
#undef AWQ_MG_Z3
    }
  }
  load_data(kb + 32 * (J + 2), st.w[BA], st.a[BA]);
  if constexpr (kAheadOpens) load_par(kb + 32 * (J + 2), st.ps0[BA], st.ps1[BA], st.pz[BA]);

  const V a = __builtin_bit_cast(V, st.a[B]);
  const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
  V ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = 1;
  // At T = 1 the MFMAs accumulate a group's blocks (P' and S over up to 128
  // rows) and the fold runs once per group; with more token rows the extra
  // 64 registers would spill, so every block folds.
  constexpr bool kAccFirst = TV == 1 ? kFirst : true;
  constexpr bool kAccLast = TV == 1 ? J % BPG == BPG - 1 : true;
  const floatx4 sx = mfma16(a, ones, kAccFirst ? zero : st.sacc);
  if constexpr (!kAccLast) st.sacc = sx;
  const uint32_t sw[8] = {st.s0.x, st.s0.y, st.s0.z, st.s0.w, st.s1.x, st.s1.y, st.s1.z, st.s1.w};
  if constexpr (BITS == 3) {
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = __builtin_amdgcn_alignbit(st.w[B][e].y, st.w[B][e].x, sh3);
      hi[e] = st.w[B][e].y >> sh3;
    }
#define AWQ_MG_CODE3(R)                                                                     \
  {                                                                                         \
    const V b = __builtin_bit_cast(                                                         \
        V, make_uint4(code3_pair<F16, R>(lo[0], hi[0], lo[1], hi[1], one),                  \
                      code3_pair<F16, R>(lo[2], hi[2], lo[3], hi[3], one),                  \
                      code3_pair<F16, R>(lo[4], hi[4], lo[5], hi[5], one),                  \
                      code3_pair<F16, R>(lo[6], hi[6], lo[7], hi[7], one)));                \
    const floatx4 p = mfma16(a, b, kAccFirst ? zero : st.pacc[R]);                          \
    if constexpr (kAccLast) {                                                               \
      const float sc = f16_to_f32(uint16_t((sw[R >> 1] >> (16 * (R & 1))) & 0xFFFFu));      \
      for (int v = 0; v < TV; ++v)                                                          \
        st.tot[R][v] = __builtin_fmaf(sc, __builtin_fmaf(-st.zf[R], sx[v], p[v]), st.tot[R][v]); \
    } else {                                                                                \
      st.pacc[R] = p;                                                                       \
    }                                                                                       \
  }
    AWQ_MG_CODE3(0) AWQ_MG_CODE3(1) AWQ_MG_CODE3(2) AWQ_MG_CODE3(3)
    AWQ_MG_CODE3(4) AWQ_MG_CODE3(5) AWQ_MG_CODE3(6) AWQ_MG_CODE3(7)
    AWQ_MG_CODE3(8) AWQ_MG_CODE3(9) AWQ_MG_CODE3(10) AWQ_MG_CODE3(11)
    AWQ_MG_CODE3(12) AWQ_MG_CODE3(13) AWQ_MG_CODE3(14) AWQ_MG_CODE3(15)
#undef AWQ_MG_CODE3
  } else {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = c ? st.w[B][e].y : st.w[B][e].x;
#define AWQ_MG_CODE(R)                                                                      \
  {                                                                                         \
    constexpr int m = c * 8 + R;                                                            \
    const V b = __builtin_bit_cast(                                                         \
        V, make_uint4(code_pair<F16, R>(w[0], w[1]), code_pair<F16, R>(w[2], w[3]),         \
                      code_pair<F16, R>(w[4], w[5]), code_pair<F16, R>(w[6], w[7])));       \
    const floatx4 p = mfma16(a, b, kAccFirst ? zero : st.pacc[m]);                          \
    if constexpr (kAccLast) {                                                               \
      const float sc = f16_to_f32(uint16_t((sw[m >> 1] >> (16 * (m & 1))) & 0xFFFFu));      \
      for (int v = 0; v < TV; ++v)                                                          \
        st.tot[m][v] = __builtin_fmaf(sc, __builtin_fmaf(-st.zf[m], sx[v], p[v]), st.tot[m][v]); \
    } else {                                                                                \
      st.pacc[m] = p;                                                                       \
    }                                                                                       \
  }
    if (c == 0) {
      constexpr int c = 0;
      AWQ_MG_CODE(0) AWQ_MG_CODE(1) AWQ_MG_CODE(2) AWQ_MG_CODE(3)
      AWQ_MG_CODE(4) AWQ_MG_CODE(5) AWQ_MG_CODE(6) AWQ_MG_CODE(7)
    } else {
      constexpr int c = 1;
      AWQ_MG_CODE(0) AWQ_MG_CODE(1) AWQ_MG_CODE(2) AWQ_MG_CODE(3)
      AWQ_MG_CODE(4) AWQ_MG_CODE(5) AWQ_MG_CODE(6) AWQ_MG_CODE(7)
    }
#undef AWQ_MG_CODE
  }
  }
}

template <bool F16, int BITS, int G, int TV>
__global__ __launch_bounds__(256, 2) void w4a16_mgemv_kernel(
    const uint16_t* __restrict__ X, int64_t T, int64_t N, int64_t K,
    const int32_t* __restrict__ qweight, const int32_t* __restrict__ qzeros,
    const uint16_t* __restrict__ scales, int kpw, float* __restrict__ partial) {
  __shared__ float red[kMgWaves][16][kMgCols * 8 + 4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int jj = lane & 15, lg = lane >> 4;
  // Words per k row, and the lane's 16 output rows n0 .. n0 + 15: 4 bits, two
  // adjacent word columns (one 8-byte load per k row); 3 bits, half of a
  // 32-row group, words 0-1 (even jj) or 1-2 (odd jj) of its 3 (two 4-byte
  // loads). Lanes past N (N a multiple of 16, or of 32 for 3 bits: whole
  // lanes, whole lane pairs) and token rows past T read column 0 / row 0
  // instead: every load stays in bounds and needs no branch, and an MFMA
  // output column depends only on its own B column (an output row on its own
  // A row), so those lanes' results, which are never stored, do not reach the
  // others.
  const int64_t RS = BITS == 4 ? N / 8 : N / 32 * 3;
  // Workgroups are dealt to the 8 XCDs in turn, and each XCD has its own L2.
  // XCD i takes a contiguous run of (column block, chunk) indices, column
  // blocks fastest, so neighbouring column blocks, whose qweight row
  // segments can share cache lines (3 bits: 96 bytes per row and block),
  // meet in one L2.
  int bx, by;
  {
    const int W = int(gridDim.x) * int(gridDim.y);
    const int id = int(blockIdx.x) + int(gridDim.x) * int(blockIdx.y);
    const int q = W / 8, r = W % 8, xi = id % 8;
    const int L = xi * q + (xi < r ? xi : r) + id / 8;
    bx = L % int(gridDim.x);
    by = L / int(gridDim.x);
  }
  const int64_t n0 = int64_t(bx) * (kMgCols * 8) + 16 * jj;
  const bool live = n0 < N;
  const int64_t nl0 = live ? n0 : 0;
  const int64_t wq = !live ? 0 : BITS == 4 ? n0 / 8 : 3 * (n0 / 32) + (jj & 1);
  // This wave's k rows: kpw (a multiple of 128) from its place in the grid,
  // cut at K (a multiple of 128); waves past K have none.
  const int kw0 = (by * kMgWaves + wave) * kpw;
  const int kw1 = kw0 + kpw < int(K) ? kw0 + kpw : int(K);
  const uint16_t* xrow = X + int64_t(jj < T ? jj : 0) * K + 8 * lg;
  const int32_t* qlane = qweight + int64_t(8 * lg) * RS + wq;
  auto load2 = [](const int32_t* p) {
    if constexpr (BITS == 4) return *reinterpret_cast<const uint2*>(p);
    else return make_uint2(uint32_t(p[0]), uint32_t(p[1]));
  };

  MgState<F16> st;
#pragma unroll
  for (int m = 0; m < kMgMfma; ++m) st.tot[m] = floatx4{0.f, 0.f, 0.f, 0.f};

  // The exponent bits of B = 1 + q/16, held in a register so that the 3-bit
  // operand's mask and or fuse into one instruction.
  uint32_t one = F16 ? 0x3C003C00u : 0x3F803F80u;
  asm volatile("" : "+v"(one));
  if (kw0 < kw1) {
    // k-blocks past the wave's last re-read its last block (a harmless
    // in-bounds prefetch)
    auto load_data = [&](int kb, uint2 (&w)[8], uint4& a) {
      const int kc = kb < kw1 ? kb : kw1 - 32;
      const int32_t* q = qlane + int64_t(kc) * RS;
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = load2(q + e * RS);
      a = *reinterpret_cast<const uint4*>(xrow + kc);
    };
    auto load_par = [&](int kb, uint4& s0, uint4& s1, uint2& z) {
      const int64_t g = (kb < kw1 ? kb : kw1 - 32) / G;
      s0 = *reinterpret_cast<const uint4*>(scales + g * N + nl0);
      s1 = *reinterpret_cast<const uint4*>(scales + g * N + nl0 + 8);
      z = load2(qzeros + g * RS + wq);
    };
    load_data(kw0, st.w[0], st.a[0]);
    load_par(kw0, st.ps0[0], st.ps1[0], st.pz[0]);
    load_data(kw0 + 32, st.w[1], st.a[1]);
    if (G == 32) load_par(kw0 + 32, st.ps0[1], st.ps1[1], st.pz[1]);
    for (int kb = kw0; kb < kw1; kb += 128) {
      mg_block<F16, BITS, G, TV, 0>(st, kb, load_data, load_par, one);
      __builtin_amdgcn_sched_barrier(0);
      mg_block<F16, BITS, G, TV, 1>(st, kb, load_data, load_par, one);
      __builtin_amdgcn_sched_barrier(0);
      mg_block<F16, BITS, G, TV, 2>(st, kb, load_data, load_par, one);
      __builtin_amdgcn_sched_barrier(0);
      mg_block<F16, BITS, G, TV, 3>(st, kb, load_data, load_par, one);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int m = 0; m < kMgMfma; ++m)
#pragma unroll
    for (int v = 0; v < TV; ++v) st.tot[m][v] *= 16.f;

  // totals -> LDS [wave][t][n_local], n_local = 16·jj + m (rows 4·lg + v
  // for v < TV: with TV < 4, T <= TV and only lane group 0's rows are read)
#pragma unroll
  for (int m = 0; m < kMgMfma; ++m)
#pragma unroll
    for (int v = 0; v < TV; ++v) red[wave][4 * lg + v][16 * jj + m] = st.tot[m][v];
  __syncthreads();
  const int nl = threadIdx.x;
  const int64_t n = int64_t(bx) * kMgCols * 8 + nl;
  if (n < N) {
    for (int t = 0; t < T; ++t) {
      const float s = ((red[0][t][nl] + red[1][t][nl]) + red[2][t][nl]) + red[3][t][nl];
      partial[(int64_t(by) * T + t) * N + n] = s;
    }
  }
}

// Y[t][n] = Σ_c partial[c][t][n], chunks added in a fixed order (lane group
// cl takes chunks cl, cl+4, ...; the four sums are then added in order),
// rounded once. 64 outputs per workgroup.
template <bool F16>
__global__ __launch_bounds__(256) void w4a16_gemv_reduce_kernel(const float* __restrict__ partial,
                                                                int64_t chunks, int64_t T,
                                                                int64_t N,
                                                                uint16_t* __restrict__ Y) {
  __shared__ float red[4][64];
  const int o = threadIdx.x & 63, cl = threadIdx.x >> 6;
  const int64_t e = int64_t(blockIdx.x) * 64 + o;
  float s = 0.f;
  if (e < T * N) {
#pragma unroll 8
    for (int64_t c = cl; c < chunks; c += 4) s += partial[c * T * N + e];
  }
  red[cl][o] = s;
  __syncthreads();
  if (cl == 0 && e < T * N) Y[e] = to16<F16>(((red[0][o] + red[1][o]) + red[2][o]) + red[3][o]);
}

template <bool F16, int TT>
void launch_gemv_t(dim3 grid, hipStream_t st, const uint16_t* X, int64_t T, int64_t N, int64_t K,
                   const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                   int group, int kpw, float* partial) {
  w4a16_gemv_kernel<F16, TT><<<grid, 256, 0, st>>>(X, T, N, K, qweight, qzeros, scales, group,
                                                   kpw, partial);
}

template <bool F16>
void launch_gemv(dim3 grid, hipStream_t st, const uint16_t* X, int64_t T, int64_t N, int64_t K,
                 const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales, int group,
                 int kpw, float* partial) {
  if (T <= 1)
    launch_gemv_t<F16, 1>(grid, st, X, T, N, K, qweight, qzeros, scales, group, kpw, partial);
  else if (T <= 2)
    launch_gemv_t<F16, 2>(grid, st, X, T, N, K, qweight, qzeros, scales, group, kpw, partial);
  else if (T <= 4)
    launch_gemv_t<F16, 4>(grid, st, X, T, N, K, qweight, qzeros, scales, group, kpw, partial);
  else if (T <= 8)
    launch_gemv_t<F16, 8>(grid, st, X, T, N, K, qweight, qzeros, scales, group, kpw, partial);
  else
    launch_gemv_t<F16, 16>(grid, st, X, T, N, K, qweight, qzeros, scales, group, kpw, partial);
}

}  // namespace

hipError_t launch_w4a16_dequant(const int32_t* qweight, const int32_t* qzeros,
                                const uint16_t* scales, int64_t N, int64_t K, int group, int f16,
                                uint16_t* Wd, hipStream_t st) {
  // 16-byte loads of 4 word columns need N a multiple of 32 and qweight
  // 16-byte aligned; otherwise one word column per lane
  if (N % 32 == 0 && (reinterpret_cast<uintptr_t>(qweight) & 15u) == 0) {
    const int64_t lanes = (K / 8) * (N / 32);
    const unsigned blocks = unsigned((lanes + 255) / 256);
    if (f16)
      dequant4x4_kernel<true><<<blocks, 256, 0, st>>>(qweight, qzeros, scales, N, K, group, Wd);
    else
      dequant4x4_kernel<false><<<blocks, 256, 0, st>>>(qweight, qzeros, scales, N, K, group, Wd);
    return hipGetLastError();
  }
  const int64_t lanes = (K / 8) * (N / 8);
  const unsigned blocks = unsigned((lanes + 255) / 256);
  if (f16)
    dequant_kernel<true><<<blocks, 256, 0, st>>>(qweight, qzeros, scales, N, K, group, Wd);
  else
    dequant_kernel<false><<<blocks, 256, 0, st>>>(qweight, qzeros, scales, N, K, group, Wd);
  return hipGetLastError();
}

// Prefill GEMM straight from the packed layer (K·N/2 < 2^31 bytes, K a
// multiple of 128, group 32, 64 or 128).
hipError_t launch_w4a16_gemm_q(const uint16_t* X, const int32_t* qweight, const int32_t* qzeros,
                               const uint16_t* scales, int64_t M, int64_t N, int64_t K,
                               int group, int f16, uint16_t* Y, hipStream_t st) {
  if (K % 128 || N % 8 || K * (N / 8) * 4 >= (int64_t(1) << 31) ||
      (group != 32 && group != 64 && group != 128))
    return hipErrorInvalidValue;
  const int gshift = group == 32 ? 5 : group == 64 ? 6 : 7;   // log2 of the group size
  const int tiles_m = int((M + BM - 1) / BM), tiles_n = int((N + BN - 1) / BN);
  const unsigned blocks = unsigned(q_gemm_blocks(tiles_m, tiles_n));
  if (f16)
    w4a16_gemm_q_kernel<true><<<blocks, NT, 0, st>>>(X, qweight, qzeros, scales, M, N, K, gshift,
                                                     tiles_m, tiles_n, Y);
  else
    w4a16_gemm_q_kernel<false><<<blocks, NT, 0, st>>>(X, qweight, qzeros, scales, M, N, K,
                                                      gshift, tiles_m, tiles_n, Y);
  return hipGetLastError();
}

hipError_t launch_w3a16_dequant(const int32_t* qweight, const int32_t* qzeros,
                                const uint16_t* scales, int64_t N, int64_t K, int group, int f16,
                                uint16_t* Wd, hipStream_t st) {
  if (N % 32 || K % 8) return hipErrorInvalidValue;
  const int64_t lanes = (K / 8) * (N / 32);
  const unsigned blocks = unsigned((lanes + 255) / 256);
  if (f16)
    dequant3_kernel<true><<<blocks, 256, 0, st>>>(qweight, qzeros, scales, N, K, group, Wd);
  else
    dequant3_kernel<false><<<blocks, 256, 0, st>>>(qweight, qzeros, scales, N, K, group, Wd);
  return hipGetLastError();
}

hipError_t launch_w4a16_gemm(const uint16_t* X, const uint16_t* Wd, int64_t M, int64_t N,
                             int64_t K, int f16, uint16_t* Y, hipStream_t st) {
  if (K % 128) return hipErrorInvalidValue;
  const int tiles_m = int((M + BM - 1) / BM), tiles_n = int((N + BN - 1) / BN);
  const unsigned blocks = unsigned(gemm_blocks(tiles_m, tiles_n));
  if (f16)
    w4a16_gemm_kernel<true><<<blocks, NT, 0, st>>>(X, Wd, M, N, K, tiles_m, tiles_n, Y);
  else
    w4a16_gemm_kernel<false><<<blocks, NT, 0, st>>>(X, Wd, M, N, K, tiles_m, tiles_n, Y);
  return hipGetLastError();
}

// 1 <= T <= 16 token rows; kpw in {32, 64, 128} with K a multiple of 4·kpw;
// partial holds (K / (4·kpw)) x T x N floats.
hipError_t launch_w4a16_gemv(const uint16_t* X, int64_t T, int64_t N, int64_t K,
                             const int32_t* qweight, const int32_t* qzeros,
                             const uint16_t* scales, int group, int f16, int64_t kpw,
                             float* partial, hipStream_t st) {
  const int64_t chunks = K / (kGemvWaves * kpw);
  dim3 grid(unsigned((N / 8 + kGemvCols - 1) / kGemvCols), unsigned(chunks));
  if (f16)
    launch_gemv<true>(grid, st, X, T, N, K, qweight, qzeros, scales, group, int(kpw), partial);
  else
    launch_gemv<false>(grid, st, X, T, N, K, qweight, qzeros, scales, group, int(kpw), partial);
  return hipGetLastError();
}

// 1 <= T <= 16 token rows; K a multiple of 128; kpw a multiple of 128;
// partial holds ceil(K / (4·kpw)) x T x N floats. 4 bits: N a multiple of
// 16, qweight and qzeros 8-byte aligned; 3 bits: N a multiple of 32.
template <bool F16, int BITS, int TV>
void launch_mgemv_tv(int group, dim3 grid, hipStream_t st, const uint16_t* X, int64_t T,
                     int64_t N, int64_t K, const int32_t* qweight, const int32_t* qzeros,
                     const uint16_t* scales, int kpw, float* partial) {
  if (group == 32)
    w4a16_mgemv_kernel<F16, BITS, 32, TV><<<grid, 256, 0, st>>>(X, T, N, K, qweight, qzeros,
                                                                scales, kpw, partial);
  else if (group == 64)
    w4a16_mgemv_kernel<F16, BITS, 64, TV><<<grid, 256, 0, st>>>(X, T, N, K, qweight, qzeros,
                                                                scales, kpw, partial);
  else
    w4a16_mgemv_kernel<F16, BITS, 128, TV><<<grid, 256, 0, st>>>(X, T, N, K, qweight, qzeros,
                                                                 scales, kpw, partial);
}

// The MFMA's output rows are token rows 4·(lane / 16) + v; with T <= 2 only
// v < T of lane group 0 are stored, so the scale and zero-point fold runs on
// TV = T rows (else all 4).
template <bool F16, int BITS>
void launch_mgemv_g(int group, dim3 grid, hipStream_t st, const uint16_t* X, int64_t T, int64_t N,
                    int64_t K, const int32_t* qweight, const int32_t* qzeros,
                    const uint16_t* scales, int kpw, float* partial) {
  if (T == 1)
    launch_mgemv_tv<F16, BITS, 1>(group, grid, st, X, T, N, K, qweight, qzeros, scales, kpw,
                                  partial);
  else if (T == 2)
    launch_mgemv_tv<F16, BITS, 2>(group, grid, st, X, T, N, K, qweight, qzeros, scales, kpw,
                                  partial);
  else
    launch_mgemv_tv<F16, BITS, 4>(group, grid, st, X, T, N, K, qweight, qzeros, scales, kpw,
                                  partial);
}

hipError_t launch_w4a16_mgemv(const uint16_t* X, int64_t T, int64_t N, int64_t K,
                              const int32_t* qweight, const int32_t* qzeros,
                              const uint16_t* scales, int group, int f16, int64_t kpw,
                              float* partial, hipStream_t st, int bits) {
  if (T < 1 || T > 16 || N % (bits == 3 ? 32 : 16) || K % 128 || kpw < 128 || kpw % 128 ||
      K > (int64_t(1) << 30) || (group != 32 && group != 64 && group != 128) ||
      (bits != 3 && bits != 4))
    return hipErrorInvalidValue;
  const int64_t chunks = (K + kMgWaves * kpw - 1) / (kMgWaves * kpw);
  dim3 grid(unsigned((N + kMgCols * 8 - 1) / (kMgCols * 8)), unsigned(chunks));
  if (bits == 3) {
    if (f16)
      launch_mgemv_g<true, 3>(group, grid, st, X, T, N, K, qweight, qzeros, scales, int(kpw),
                              partial);
    else
      launch_mgemv_g<false, 3>(group, grid, st, X, T, N, K, qweight, qzeros, scales, int(kpw),
                               partial);
  } else if (f16) {
    launch_mgemv_g<true, 4>(group, grid, st, X, T, N, K, qweight, qzeros, scales, int(kpw),
                            partial);
  } else {
    launch_mgemv_g<false, 4>(group, grid, st, X, T, N, K, qweight, qzeros, scales, int(kpw),
                             partial);
  }
  return hipGetLastError();
}

hipError_t launch_w4a16_gemv_reduce(const float* partial, int64_t chunks, int64_t T, int64_t N,
                                    int f16, uint16_t* Y, hipStream_t st) {
  const unsigned rblocks = unsigned((T * N + 63) / 64);
  if (f16)
    w4a16_gemv_reduce_kernel<true><<<rblocks, 256, 0, st>>>(partial, chunks, T, N, Y);
  else
    w4a16_gemv_reduce_kernel<false><<<rblocks, 256, 0, st>>>(partial, chunks, T, N, Y);
  return hipGetLastError();
}

}  // namespace awq
