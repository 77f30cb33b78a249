// The search's output errors through the Gram matrix of the activations:
//
//   M_n = Σ_t (Σ_k X[t][k]·E[n][k])² = E_n · G · E_nᵀ,   G = XᵀX  [K, K]
//
// (an exact identity of the error the pages measure: "05 — AWQ: Activation-
// Aware Weight Scaling", section 4, quantise and measure the output MSE).
// G costs 2·T·K² once per layer; each candidate row then costs 2·K² instead
// of 2·T·K, T/K times less (16x at 64K tokens and K = 4096).
//
//  1. gram_partial_kernel: G is symmetric, so only its 256x256 tiles on and
//     above the diagonal are formed, on the MFMA schedule of gemm_core.h
//     with its operands read from X itself: k-tiles of 64 tokens x 256
//     channels go to LDS as they are, and transposing LDS reads
//     (ds_read_b64_tr_b16) hand each lane its channel's 8 consecutive tokens.
//     To keep every CU busy the token range is split into S slices of whole
//     64-token k-tiles, slice s taking k-tiles [s·KT/S, (s+1)·KT/S) (S chosen
//     on the host to balance whole rounds of work: at 64K tokens and
//     K = 4096, 15 slices of 68 or 69 k-tiles make 2040 units, 8 rounds of
//     256 CUs); each (tile, slice) unit stores its float32 partial tile.
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
//  2. gram_search_kernel: for a batch of candidate error rows E [Nc, K]
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
// 2. G = XᵀX: upper tiles x token slices, then the slice sum as hi/lo halves
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

// Upper tile q in row-pair order -> (tm, tn): pair p is row p (tiles p ..
// nt - 1) then row nt - 1 - p (its nt - p .. nt - 1 tiles follow), nt + 1
// tiles a pair; a pair needs only the panels from row p up.
__device__ __forceinline__ void pair_tile(int q, int nt, int& tm, int& tn) {
  const int p = q / (nt + 1), r = q - p * (nt + 1);
  if (r < nt - p) {
    tm = p;
    tn = p + r;
  } else {
    tm = nt - 1 - p;
    tn = tm + (r - (nt - p));
  }
}

// An operand k-tile is 64 tokens x 256 channels of X, 64 rows of 512 bytes
// (32 chunks of 16 bytes) in one ring array, chunk c of token row r at c ^
// hx(r). One ds_read_b64_tr_b16 returns lane l (of each 16-lane group) the
// l-th of the 16 elements that the group's quad e (lanes 4e .. 4e+3, 8 bytes
// each) points at, for e = 0..3: four token rows of one channel. An MFMA
// operand (8 tokens of one channel per lane) is two such reads. The 16 rows
// one read touches (4 per group, the groups 8 rows apart) differ in bits 0,
// 1, 3 and 4, so hx takes those bits: their 32-byte runs land on 16
// distinct chunk pairs.
__device__ __forceinline__ int hx(int r) { return 2 * ((r & 3) | ((r >> 1) & 12)); }
constexpr int kXOob = 0x40000000;   // a byte offset past any k-tile's records

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // one MFMA operand

struct XCtx {
  const uint16_t* a;   // X + t0·K + m0: row-side channels
  const uint16_t* b;   // X + t0·K + n0: column-side channels
  int64_t K;           // X's row length (elements)
  int tokens;          // tokens from t0 to the end of X
  int ca, cb;          // valid channels from m0 and from n0 (128 or 256)
  int KT;              // k-tiles of the slice
  int wave;
  int vbA[2], vbB[2];  // copy j's per-lane byte offset within its k-tile, by j & 1
  int rdA[8], rdB[8];  // fragment block i's per-lane LDS byte offset (k-step 0, rows 0-3)
};

// Buffer resource over k-tile kt of one operand: 64 token rows from
// base + 64·kt·K, ending at the last valid channel of the last valid token
// (nothing past it, and nothing at all past X's last token).
// (Every input is the same on all lanes; readfirstlane says so to the
// compiler, which otherwise wraps each copy in a loop over distinct values.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t xtile_rsrc(const uint16_t* base, int64_t K,
                                                             int tokens, int chans, int kt) {
  int rows = tokens - 64 * kt;
  rows = rows < 0 ? 0 : rows > 64 ? 64 : rows;
  const int rec = __builtin_amdgcn_readfirstlane(int(rows ? (int64_t(rows - 1) * K + chans) * 2 : 0));
  const uint64_t p = reinterpret_cast<uint64_t>(base + int64_t(64) * kt * K);
  const uint64_t pu = (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(p >> 32)))) << 32) |
                      uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(p))));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<uint16_t*>(pu), 0, rec, 0x00020000);
}

__device__ __forceinline__ void xctx_setup(XCtx& c) {
  const int lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: LDS targets in SGPRs
  // copy j of wave w fills token rows r0 = 8w + 32·(j / 4) + 2·(j % 4) and
  // r0 + 1 (lane / 32), physical chunk lane % 32; hx of those rows depends
  // on j only through j & 1
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int r = 8 * c.wave + 2 * jj + (lane >> 5);
    const int ch = (lane & 31) ^ hx(r);               // logical chunk: channels 8·ch ..
    const int64_t row_bytes = int64_t(8 * c.wave + (lane >> 5)) * c.K * 2;
    c.vbA[jj] = 8 * ch < c.ca ? int(row_bytes) + 16 * ch : kXOob;
    c.vbB[jj] = 8 * ch < c.cb ? int(row_bytes) + 16 * ch : kXOob;
  }
  // fragment reads: group g = lane / 16 takes tokens 8g .. 8g+7 of a k-step,
  // quad q = (lane / 4) % 4 the rows 8g + q (and + 4), lane j4 = lane % 4 the
  // channels 4·j4 .. +3 of the block's 16
  const int g = lane >> 4, q = (lane >> 2) & 3, j4 = lane & 3;
  const int h = 2 * (q | (g << 2));
  const int wm = c.wave >> 1, wn = c.wave & 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    c.rdA[i] = (8 * g + q) * 512 + (((16 * wm + 2 * i) ^ h) + (j4 >> 1)) * 16 + (j4 & 1) * 8;
    c.rdB[i] = (8 * g + q) * 512 + (((16 * wn + 2 * i) ^ h) + (j4 >> 1)) * 16 + (j4 & 1) * 8;
  }
}

template <int S>
__device__ __forceinline__ void xcopy(const XCtx& c, __amdgpu_buffer_rsrc_t rsA,
                                      __amdgpu_buffer_rsrc_t rsB, int q) {
  // copy q of the 16 a wave issues per k-tile: A's 8, then B's 8
  const int j = q & 7;
  const int r0 = 8 * c.wave + 32 * (j >> 2) + 2 * (j & 3);
  const int soff = int((32 * (j >> 2) + 2 * (j & 3)) * c.K * 2);
  if (q < 8)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, AWQ_LDS(stage64_a<S>() + r0 * 32), 16,
                                             c.vbA[j & 1], soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, AWQ_LDS(stage64_b<S>() + r0 * 32), 16,
                                             c.vbB[j & 1], soff, 0, 0);
}

__device__ __forceinline__ u32x2 tr_read(const uint4* stage, int byte_off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(reinterpret_cast<const char*>(stage) + byte_off)));
}
// half-read r (0..31) of k-step ks: fragment r / 2 (B blocks 0..7, then A
// blocks), token rows + 4·(r % 2)
template <int S>
__device__ __forceinline__ void xfrag(const XCtx& c, int ks, int r, u32x4 (&fa)[8], u32x4 (&fb)[8]) {
  const int f = r >> 1, hh = r & 1;
  const int row_off = (32 * ks + 4 * hh) * 512;
  // tokens 0-3 of the lane's 8 go to words 0-1, tokens 4-7 to words 2-3
  auto put = [hh](u32x4& dst, u32x2 v) {
    const u32x4 w = __builtin_shufflevector(v, v, 0, 1, 0, 1);
    dst = hh ? __builtin_shufflevector(dst, w, 0, 1, 6, 7) : __builtin_shufflevector(dst, w, 4, 5, 2, 3);
  };
  if (f < 8)
    put(fb[f], tr_read(stage64_b<S>(), c.rdB[f] + row_off));
  else
    put(fa[f - 8], tr_read(stage64_a<S>(), c.rdA[f - 8] + row_off));
}
__device__ __forceinline__ bf16x8_t as_bf16(const u32x4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// One 64-token k-tile, the schedule of region16 with two half-reads where it
// has one read: the previous k-step's 64 MFMAs carry k-step 0's 32
// half-reads and the next k-tile's 16 copies; k-step 0's carry k-step 1's.
template <int S, bool PREV>
__device__ __forceinline__ void xregion(const XCtx& c, int kt, floatx4 (&acc)[8][8],
                                        u32x4 (&f0a)[8], u32x4 (&f0b)[8], u32x4 (&f1a)[8],
                                        u32x4 (&f1b)[8]) {
  const bool more = kt + 1 < c.KT;
  const __amdgpu_buffer_rsrc_t rsA = xtile_rsrc(c.a, c.K, more ? c.tokens : 0, c.ca, kt + 1);
  const __amdgpu_buffer_rsrc_t rsB = xtile_rsrc(c.b, c.K, more ? c.tokens : 0, c.cb, kt + 1);
  if (PREV) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int i = q >> 1, j0 = (q & 1) * 4;
      mfma16(acc[i][j0], as_bf16(f1a[i]), as_bf16(f1b[j0]));
      xfrag<S>(c, 0, 2 * q, f0a, f0b);
      mfma16(acc[i][j0 + 1], as_bf16(f1a[i]), as_bf16(f1b[j0 + 1]));
      xfrag<S>(c, 0, 2 * q + 1, f0a, f0b);
      mfma16(acc[i][j0 + 2], as_bf16(f1a[i]), as_bf16(f1b[j0 + 2]));
      xcopy<S ^ 1>(c, rsA, rsB, q);
      mfma16(acc[i][j0 + 3], as_bf16(f1a[i]), as_bf16(f1b[j0 + 3]));
    }
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q) xcopy<S ^ 1>(c, rsA, rsB, q);
#pragma unroll
    for (int r = 0; r < 32; ++r) xfrag<S>(c, 0, r, f0a, f0b);
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = q >> 1, j0 = (q & 1) * 4;
    mfma16_acc<!PREV>(acc[i][j0], as_bf16(f0a[i]), as_bf16(f0b[j0]));
    xfrag<S>(c, 1, 2 * q, f1a, f1b);
    mfma16_acc<!PREV>(acc[i][j0 + 1], as_bf16(f0a[i]), as_bf16(f0b[j0 + 1]));
    xfrag<S>(c, 1, 2 * q + 1, f1a, f1b);
    mfma16_acc<!PREV>(acc[i][j0 + 2], as_bf16(f0a[i]), as_bf16(f0b[j0 + 2]));
    mfma16_acc<!PREV>(acc[i][j0 + 3], as_bf16(f0a[i]), as_bf16(f0b[j0 + 3]));
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  region_barrier();
}

// Units v = s·U + q (slice s, upper tile q). With compact (from 1024 units
// on), runs of 32 consecutive units go to one XCD (consecutive block ids go
// round-robin over the 8 XCDs: block b runs on XCD b % 8, the i-th there
// for i = b / 8) and tiles follow the row-pair order, so an XCD's 32
// concurrent tiles draw on ~15 panels of one slice instead of 32 panel-slices
// of two (at K = 4096); otherwise block v is unit v in row-major tile order.
// P[(s·U + u)][256·256]: float32 partial tile of row-major upper tile u.
// X [T, K] row-major; tokens past T read as zero.
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gram_partial_kernel(const uint16_t* __restrict__ X, int64_t T, int64_t K, int64_t KT,
                           int S, int nt, int U, int compact, float* __restrict__ P) {
  int64_t v = blockIdx.x;
  if (compact) {
    const int b = int(blockIdx.x), x = b & 7, i = b >> 3;
    v = int64_t(i >> 5) * 256 + 32 * x + (i & 31);
    if (v >= int64_t(U) * S) return;
  }
  const int s = int(v / U), q = int(v % U);
  int tm, tn, u = q;
  if (compact) {
    pair_tile(q, nt, tm, tn);
    u = tm * nt - tm * (tm - 1) / 2 + (tn - tm);
  } else {
    upper_tile(q, nt, tm, tn);
  }
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;
  const int64_t k0 = int64_t(s) * KT / S, k1 = int64_t(s + 1) * KT / S;
  const int64_t t0 = k0 * BK64;
  XCtx c;
  c.K = K;
  c.a = X + t0 * K + m0;
  c.b = X + t0 * K + n0;
  c.tokens = int(T - t0 < int64_t(1) << 30 ? T - t0 : int64_t(1) << 30);
  c.ca = int(K - m0 < BM ? K - m0 : BM);
  c.cb = int(K - n0 < BN ? K - n0 : BN);
  c.KT = int(k1 - k0);
  xctx_setup(c);

  // k-tile 0 into stage 0
  {
    const __amdgpu_buffer_rsrc_t rsA = xtile_rsrc(c.a, K, c.tokens, c.ca, 0);
    const __amdgpu_buffer_rsrc_t rsB = xtile_rsrc(c.b, K, c.tokens, c.cb, 0);
#pragma unroll
    for (int qq = 0; qq < 16; ++qq) xcopy<0>(c, rsA, rsB, qq);
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  region_barrier();
  floatx4 acc[8][8];
  u32x4 f0a[8], f0b[8], f1a[8], f1b[8];
  xregion<0, false>(c, 0, acc, f0a, f0b, f1a, f1b);
  int kt = 1;
  for (; kt + 1 < c.KT; kt += 2) {
    xregion<1, true>(c, kt, acc, f0a, f0b, f1a, f1b);
    xregion<0, true>(c, kt + 1, acc, f0a, f0b, f1a, f1b);
  }
  if (kt < c.KT) xregion<1, true>(c, kt, acc, f0a, f0b, f1a, f1b);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) mfma16(acc[i][j], as_bf16(f1a[i]), as_bf16(f1b[j]));
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(acc[i][j]));

  // Store through LDS: lane l of block (i, j) holds column 16·j + l % 16
  // and rows 16·i + 4·(l/16) + v of the wave's 128 x 128, scattered over
  // half-lines if stored as they lie. The k-loop left the ring idle (its
  // last region ended on a barrier after its reads and copies), so each
  // wave takes one of its four 32 KiB arrays, writes 64 of its columns
  // there as 128 rows of 64 floats, reads them back 4 consecutive floats
  // per lane and stores whole 256-byte row runs; twice. Column c of row r
  // sits at c ^ (16·((r / 4) % 4)): the 64 lanes of a 4-byte write (4 rows
  // 4 apart, 16 columns) land on 64 distinct banks, and the 4 floats a
  // 16-byte read takes stay consecutive. Only the wave itself touches its
  // array, and a wave's LDS operations take effect in order.
  const int lane = threadIdx.x & 63;
  const int wm = c.wave >> 1, wn = c.wave & 1;
  float* stg = reinterpret_cast<float*>(c.wave == 0 ? s64A0 : c.wave == 1 ? s64A1
                                        : c.wave == 2 ? s64B0 : s64B1);
  float* tile = P + (int64_t(s) * U + u) * (BM * BN) + int64_t(wm) * 128 * BN + wn * 128;
  const int rq = lane >> 4, cl = lane & 15;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
          const int r = 16 * i + 4 * rq + vv;
          stg[r * 64 + ((16 * j + cl) ^ (16 * rq))] = acc[i][4 * p + j][vv];
        }
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int r = 4 * k + rq;
      const float4 v4 = *reinterpret_cast<const float4*>(stg + r * 64 + ((4 * cl) ^ (16 * (k & 3))));
      *reinterpret_cast<float4*>(tile + int64_t(r) * BN + 64 * p + 4 * cl) = v4;
    }
  }
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

// The epilogue's block of E, E[n0 .. n0 + 255][m0 .. m0 + 255], in four
// 64-column quarters, each laid out like a B k-tile (swz64 rows of 128 bytes)
// in one of the k-tile ring's four arrays; and its column sums.
__device__ __forceinline__ uint4* e_quarter(int q) {
  return q == 0 ? s64A0 : q == 1 ? s64A1 : q == 2 ? s64B0 : s64B1;
}
__shared__ float sRedG[2 * BN];

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
#pragma nounroll
  for (int h = 0; h < n_half; ++h) {
    const int tm = h ? tiles_m - 1 - p : p;
    const int64_t m0 = int64_t(tm) * BM;
    const int64_t rows_a = K - m0 < BM ? K - m0 : BM;
    GemmCtx64 c;
    gemm_setup64(c, Gs + m0 * ldg + 2 * m0, rows_a, ldg, E + n0 * K + m0, rows_b, K,
                 2 * (K - m0), true);
    // from the last k-tile down: the row tiles of one candidate tile start at
    // different columns (256·tm) but end at the same one, so run this way
    // the workgroups of an XCD read the same E k-tiles at the same time
    c.rev = true;
    floatx4 acc[8][8];
    gemm_mainloop16<false>(c, acc);

    // Epilogue. The k-loop's reads and copies are complete (its last region
    // waited for them before its barrier), so the ring is free: copy the E
    // block into it, through a resource that ends at the tile's last valid
    // element (rows_a is 128 or 256, so whole quarters are valid or not).
    const __amdgpu_buffer_rsrc_t rsE = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(E + n0 * K + m0), 0, int(((rows_b - 1) * K + rows_a) * 2),
        0x00020000);
    const int nq = int(rows_a >> 6);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < nq) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsE, AWQ_LDS(e_quarter(q) + (c.wave * 8 + j) * 64),
                                                   16, c.vbaseB[j & 1] + 128 * q, j * c.stepB, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    __syncthreads();
    // lane l of block (i, j) holds column n = wn·128 + 16·j + l % 16 of the
    // tile and the 4 consecutive rows 4·(l/16) + v of the wave's 16-row block
    // i, whose E values are one 8-byte LDS read: quarter 2·wm + i/4, chunk
    // 2·(i % 4) + (l/16)/2 of row n, half (l/16) % 2 of it. Rows past K
    // (rows_a = 128) are skipped; columns past Nc read zeros.
    const int wm = __builtin_amdgcn_readfirstlane(c.wave >> 1), wn = c.wave & 1;
    const int lq = lane >> 4;
    // rows_a is 128 or 256: with 128 the upper wave row lies past K. Its
    // quarters were not copied, so its sums are dropped, not its reads.
    const bool rows_ok = wm == 0 || rows_a == BM;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int nl = wn * 128 + j * 16 + (lane & 15);
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4* qa = e_quarter(2 * wm + (i >> 2));
        const uint2 ev = *reinterpret_cast<const uint2*>(
            reinterpret_cast<const char*>(qa + swz64(nl, 2 * (i & 3) + (lq >> 1))) + 8 * (lq & 1));
        s = __builtin_fmaf(acc[i][j][0], __uint_as_float(ev.x << 16), s);
        s = __builtin_fmaf(acc[i][j][1], __uint_as_float(ev.x & 0xFFFF0000u), s);
        s = __builtin_fmaf(acc[i][j][2], __uint_as_float(ev.y << 16), s);
        s = __builtin_fmaf(acc[i][j][3], __uint_as_float(ev.y & 0xFFFF0000u), s);
      }
      s = rows_ok ? s : 0.f;
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (lane < 16) sRedG[wm * BN + wn * 128 + j * 16 + lane] = s;
      // one column block at a time: keeps the LDS reads from being hoisted
      // past the VGPR budget
      __builtin_amdgcn_sched_barrier(0);
    }
    // every wave's E reads come before its column sums, so past this
    // barrier the next k-loop may refill the ring
    __syncthreads();
    const int64_t col = n0 + tid;
    if (col < Nc) partials[int64_t(tm) * Nc + col] = sRedG[tid] + sRedG[BN + tid];
  }
}

}  // namespace

// S token slices of whole 64-token k-tiles (at least one each) of the Tp
// tokens (T rounded up to 128; those past T read as zero); P holds S x
// (upper tiles) float32 partial tiles of 256 x 256.
hipError_t launch_gram_build(const void* X, int64_t T, int64_t K, int64_t Tp, int S, float* P,
                             int64_t ldg, uint16_t* Gs, hipStream_t st) {
  if (K % 128 || Tp % 128 || Tp < T || S < 1 || int64_t(S) * 64 > Tp || ldg < 2 * K || ldg % 8)
    return hipErrorInvalidValue;
  const int nt = int((K + BM - 1) / BM);
  const int U = nt * (nt + 1) / 2;
  const int64_t units = int64_t(U) * S;
  const int compact = units >= 1024;
  const int64_t pblocks = compact ? (units + 255) / 256 * 256 : units;
  gram_partial_kernel<<<unsigned(pblocks), NT, 0, st>>>(static_cast<const uint16_t*>(X), T, K,
                                                        Tp / BK64, S, nt, U, compact, P);
  hipError_t e;
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
