// MFMA throughput with the search GEMM's operand pattern: 4 A and 4 B fragments of random
// bf16 per k-step, 16 accumulators, fragments rotated every k-step (register operands only).
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k(const uint4* src, float* out, int iters) {
  bf16x8_t a[2][4], b[2][4];
  for (int s = 0; s < 2; ++s)
    for (int i = 0; i < 4; ++i) {
      a[s][i] = __builtin_bit_cast(bf16x8_t, src[(blockIdx.x * 256 + threadIdx.x) * 16 + s * 8 + i]);
      b[s][i] = __builtin_bit_cast(bf16x8_t, src[(blockIdx.x * 256 + threadIdx.x) * 16 + s * 8 + 4 + i]);
    }
  floatx16 acc[4][4];
  for (int i = 0; i < 4; ++i) for (int j = 0; j < 4; ++j) for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s][i], b[s][j], acc[i][j], 0, 0, 0);
  }
  float t = 0.f;
  for (int i = 0; i < 4; ++i) for (int j = 0; j < 4; ++j) for (int v = 0; v < 16; ++v) t += acc[i][j][v];
  if (t == 1.2345f) out[0] = t;
}
__global__ void fill(uint16_t* p, int64_t n) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i < n; i += int64_t(gridDim.x) * blockDim.x) {
    uint32_t h = uint32_t(i) * 2654435761u; h ^= h >> 13; h *= 0x5bd1e995u; h ^= h >> 15;
    p[i] = uint16_t(__float_as_uint(float(h & 0xFFFF) / 65536.f - 0.5f) >> 16);
  }
}
int main() {
  uint4* src; float* out; hipMalloc(&src, 256 * 256 * 16 * 16); hipMalloc(&out, 4);
  fill<<<1024, 256>>>((uint16_t*)src, 256LL * 256 * 16 * 8); hipDeviceSynchronize();
  hipEvent_t e0, e1; hipEventCreate(&e0); hipEventCreate(&e1);
  const int iters = 10000;
  for (int pass = 0; pass < 3; ++pass) {
    hipEventRecord(e0); k<<<256, 256>>>(src, out, iters); hipEventRecord(e1); hipEventSynchronize(e1);
    float ms; hipEventElapsedTime(&ms, e0, e1);
    double fl = 256.0 * 4 * iters * 32 * 32768.0;
    printf("random operands, 1 wave/SIMD: %.1f TFLOP/s (%.1f%% of 2500), %.1f ms\n", fl / ms / 1e9, fl / ms / 1e9 / 25, ms);
  }
  return 0;
}
