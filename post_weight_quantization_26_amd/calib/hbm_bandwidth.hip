// HBM streaming bandwidth on MI355X: what a read-only stream (the shape of
// the activation-statistics pass) and a read+write stream (the shape of the
// pack and transpose passes) can reach, to set the practical ceiling the
// HBM-bound kernels are judged against.
//
// read<U, NT>: each lane loads U independent 16-byte vectors per iteration
// (grid-stride over a 4 GiB buffer) and folds them into an XOR so nothing is
// optimised away; NT = 1 uses non-temporal loads. copy: 16-byte loads and
// stores, U per iteration.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                   \
  do {                                                                             \
    hipError_t e = (x);                                                            \
    if (e != hipSuccess) {                                                         \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e));                  \
      std::exit(1);                                                                \
    }                                                                              \
  } while (0)

template <int U, int NT>
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ p, size_t n,
                                                   uint32_t* __restrict__ sink) {
  const size_t stride = size_t(gridDim.x) * 256 * U;
  uint32_t acc = 0;
  for (size_t i = size_t(blockIdx.x) * 256 * U + threadIdx.x; i < n; i += stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + size_t(u) * 256;
      if (j < n) {
        if (NT) {
          typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
          const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + j));
          v[u] = make_uint4(t.x, t.y, t.z, t.w);
        } else {
          v[u] = p[j];
        }
      } else {
        v[u] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x12345678u) sink[threadIdx.x] = acc;  // practically never true
}

template <int U>
__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ p, uint4* __restrict__ q,
                                                   size_t n) {
  const size_t stride = size_t(gridDim.x) * 256 * U;
  for (size_t i = size_t(blockIdx.x) * 256 * U + threadIdx.x; i < n; i += stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + size_t(u) * 256;
      v[u] = j < n ? p[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + size_t(u) * 256;
      if (j < n) q[j] = v[u];
    }
  }
}

template <class F>
float time_ms(F&& launch, int reps) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  launch();
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(a));
  for (int r = 0; r < reps; ++r) launch();
  CHECK(hipEventRecord(b));
  CHECK(hipEventSynchronize(b));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, a, b));
  CHECK(hipEventDestroy(a));
  CHECK(hipEventDestroy(b));
  return ms / reps;
}

template <int U, int NT>
void run_read(const uint4* p, size_t n, uint32_t* sink, int blocks_per_cu) {
  const int blocks = 256 * blocks_per_cu;
  const float ms = time_ms([&] { read_kernel<U, NT><<<blocks, 256>>>(p, n, sink); }, 10);
  std::printf("read  U=%d nt=%d blocks/CU=%2d : %7.3f ms  %6.2f TB/s\n", U, NT, blocks_per_cu, ms,
              n * 16.0 / (ms * 1e-3) / 1e12);
}

template <int U>
void run_copy(const uint4* p, uint4* q, size_t n, int blocks_per_cu) {
  const int blocks = 256 * blocks_per_cu;
  const float ms = time_ms([&] { copy_kernel<U><<<blocks, 256>>>(p, q, n); }, 10);
  std::printf("copy  U=%d       blocks/CU=%2d : %7.3f ms  %6.2f TB/s (read+write)\n", U,
              blocks_per_cu, ms, 2.0 * n * 16.0 / (ms * 1e-3) / 1e12);
}

int main() {
  const size_t bytes = size_t(4) << 30;
  const size_t n = bytes / 16;
  uint4 *p = nullptr, *q = nullptr;
  uint32_t* sink = nullptr;
  CHECK(hipMalloc(&p, bytes));
  CHECK(hipMalloc(&q, bytes / 2));
  CHECK(hipMalloc(&sink, 256 * sizeof(uint32_t)));
  CHECK(hipMemset(p, 1, bytes));
  for (int bpc : {4, 8, 16}) {
    run_read<1, 0>(p, n, sink, bpc);
    run_read<4, 0>(p, n, sink, bpc);
    run_read<8, 0>(p, n, sink, bpc);
    run_read<4, 1>(p, n, sink, bpc);
  }
  for (int bpc : {4, 8}) {
    run_copy<2>(p, q, n / 2, bpc);
    run_copy<4>(p, q, n / 2, bpc);
  }
  CHECK(hipFree(p));
  CHECK(hipFree(q));
  CHECK(hipFree(sink));
  return 0;
}
