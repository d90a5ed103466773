// Measurement aids for bench.py, not part of libspecprefill: the practical
// read bandwidth against which the scoring kernel's is compared (next to the
// 8 TB/s peak).
//
// k_read: a plain streaming read. Every lane reads 16-byte vectors,
// consecutive across the lanes of a wave, eight loads in flight per lane,
// grid-stride over the buffer.
// k_read_heads: a K cache laid out [layer][key][KV head][head_dim] read in
// the scoring kernel's order: problem by problem (layer, then KV head), the
// head's segment of every key row, blocks owning keys in groups dealt
// round-robin. No compute, no exchange: what this access pattern reaches.
// Both fold the values with XOR so that the loads cannot be dropped.
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

// Keys per block and pass: kThreads / seg16 rows, one 16-byte chunk of a
// row's head segment per lane (seg16 chunks per segment, 8 or 16).
__global__ __launch_bounds__(kThreads) void k_read_heads(const u32x4 *__restrict__ p, int n_layers,
                                                         int64_t n_keys, int hkv, int seg16,
                                                         unsigned *__restrict__ out) {
  const int rows = kThreads / seg16, r = threadIdx.x / seg16, c = threadIdx.x % seg16;
  const int64_t row16 = (int64_t)hkv * seg16;
  const int64_t step = (int64_t)gridDim.x * rows;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int y = 0; y < n_layers * hkv; ++y) {
    const int l = y / hkv, g = y % hkv;
    const u32x4 *base = p + (int64_t)l * n_keys * row16 + g * seg16 + c;
    int64_t k = (int64_t)blockIdx.x * rows + r;
    for (; k + 3 * step < n_keys; k += 4 * step) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(base + (k + u * step) * row16);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc ^= v[u];
    }
    for (; k < n_keys; k += step) acc ^= base[k * row16];
  }
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

// Reads a K cache of n_layers x n_keys rows of hkv segments of seg_bytes
// each (a multiple of 16, its count of 16-byte chunks dividing 512) once,
// problem by problem, with `blocks` blocks; `flag` is a device word the
// kernel may write. Returns a hipError_t value.
extern "C" int spbench_read_heads(const void *k, int n_layers, int64_t n_keys, int hkv,
                                  int seg_bytes, unsigned *flag, int blocks, void *stream) {
  if (n_layers < 1 || n_keys < 1 || hkv < 1 || blocks < 1 || seg_bytes % 16 != 0 ||
      seg_bytes / 16 < 1 || kThreads % (seg_bytes / 16) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read_heads, dim3(blocks), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const u32x4 *>(k),
                     n_layers, n_keys, hkv, seg_bytes / 16, flag);
  return (int)hipGetLastError();
}
