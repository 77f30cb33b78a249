// L2 -> CU streaming bandwidth: every block on an XCD re-reads the same 2 MiB window
// (L2 resident) with 16-byte-per-lane buffer loads; reports aggregate bytes/s.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
#define CHECK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e), __LINE__); return 1;} } while (0)
#define LDSP(p) ((__attribute__((address_space(3))) void*)(p))
__shared__ uint4 sbuf[4096];
template <int MODE>
__global__ __launch_bounds__(256) void stream(const uint4* __restrict__ src, int iters, uint4* out) {
  const int xcd = blockIdx.x & 7;
  const uint4* base = src + size_t(xcd) * (2 << 20) / 16;     // 2 MiB window per XCD
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, 2 << 20, 0x00020000);
  uint4 acc = make_uint4(0, 0, 0, 0);
  int off = ((blockIdx.x >> 3) * 8192 + threadIdx.x * 16) & ((2 << 20) - 1);
  for (int it = 0; it < iters; ++it) {
    if (MODE == 0) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (off + u * 4096) & ((2 << 20) - 1), 0, 0));
#pragma unroll
      for (int u = 0; u < 8; ++u) { acc.x ^= v[u].x; acc.y ^= v[u].y; acc.z ^= v[u].z; acc.w ^= v[u].w; }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDSP(sbuf + ((threadIdx.x >> 6) * 8 + u) * 64), 16, (off + u * 4096) & ((2 << 20) - 1), 0, 0, 0);
      __builtin_amdgcn_s_waitcnt(0);
    }
    off = (off + 32768) & ((2 << 20) - 1);
  }
  if (MODE == 1) acc = sbuf[threadIdx.x];
  if (acc.x == 0x12345678) out[0] = acc;
}
int main() {
  uint4 *src, *out; CHECK(hipMalloc(&src, 16 << 20)); CHECK(hipMalloc(&out, 64)); CHECK(hipMemset(src, 1, 16 << 20));
  hipEvent_t a, b; hipEventCreate(&a); hipEventCreate(&b);
  for (int blocksPerCU : {1, 2}) {
    int blocks = 256 * blocksPerCU, iters = 2000;
    for (int mode = 0; mode < 2; ++mode) {
      auto k = mode == 0 ? stream<0> : stream<1>;
      k<<<blocks, 256>>>(src, 10, out); CHECK(hipDeviceSynchronize());
      hipEventRecord(a); k<<<blocks, 256>>>(src, iters, out); hipEventRecord(b); hipEventSynchronize(b);
      float ms; hipEventElapsedTime(&ms, a, b);
      double bytes = double(blocks) * 256 * 16 * 8 * iters;
      printf("%s, %d block(s)/CU: %.2f TB/s (%.1f B/clk/CU at 2.4 GHz)\n", mode ? "buffer->LDS" : "buffer->VGPR", blocksPerCU, bytes / ms / 1e9, bytes / (ms * 1e-3) / 2.4e9 / 256);
    }
  }
  return 0;
}
