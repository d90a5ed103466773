// Measurement aid for bench.py, not part of libspecprefill: a plain
// streaming read of a device buffer, the practical read bandwidth against
// which the scoring kernel's is compared (next to the 8 TB/s peak).
//
// Every lane reads 16-byte vectors, consecutive across the lanes of a wave,
// eight loads in flight per lane, grid-stride over the buffer; the values
// are folded with XOR so that the loads cannot be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 512;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void k_read(const u32x4 *__restrict__ p, size_t n16,
                                                   unsigned *__restrict__ out) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) out[0] = 1u;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from `buf` once; `flag` is a device word
// the kernel may write. Blocks: `blocks_per_cu` per compute unit. Returns a
// hipError_t value.
extern "C" int spbench_read(const void *buf, size_t bytes, unsigned *flag, int blocks_per_cu,
                            void *stream) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  if (bytes % 16 != 0 || blocks_per_cu < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read, dim3(cus * blocks_per_cu), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const u32x4 *>(buf), bytes / 16, flag);
  return (int)hipGetLastError();
}
