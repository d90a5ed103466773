// Chunk selection: fixed top-p or cumulative attention mass, per prompt.
//
// Method: "Speculative prefill" (llama.cpp pull request 27692), Approach
// step 4 (keep the top-p fraction of chunks plus BOS and the prompt
// boundary); "SpecPrefill — Implementation Guide", v3 Improvements item 1
// (sort chunks by score and keep them from the highest down until the kept
// share of the total attention mass reaches the threshold).
//
// One 1024-thread block per prompt. Each chunk gets a 64-bit key
//   (~ordered(score) << 32) | (index + 1)
// so an ascending sort visits chunks by score, highest first, and equal
// scores by lower index; the final chunk gets key 0 and comes first (it is
// always kept). A bitonic sort of the keys runs in LDS; top-p then keeps the
// first kc sorted chunks, and mass mode finds the first sorted position whose
// fp64 prefix sum reaches mass * total (fixed-order block scan).
#include <limits.h>

#include "sp_internal.h"

namespace sp {
namespace {

constexpr int kSelThreads = 1024;

__device__ __forceinline__ uint64_t chunk_key(float v, int i) {
  const unsigned u = __float_as_uint(v);
  const unsigned ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // ascending in v
  return ((uint64_t)(~ord) << 32) | (uint64_t)(unsigned)(i + 1);
}

__device__ __forceinline__ float key_score(uint64_t key) {
  const unsigned ord = ~(unsigned)(key >> 32);
  const unsigned u = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
  return __uint_as_float(u);
}

__global__ __launch_bounds__(kSelThreads) void k_select(int mode, double param, SegTable chunks,
                                                        SelectBudget budget, int p2,
                                                        const float *__restrict__ cs,
                                                        uint8_t *__restrict__ keep,
                                                        int32_t *__restrict__ n_kept) {
  extern __shared__ uint64_t keys[];
  __shared__ double part[kSelThreads];
  __shared__ int found;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int c0 = chunks.unit_off[b], nc = chunks.unit_off[b + 1] - c0;
  for (int i = tid; i < p2; i += kSelThreads) {
    uint64_t key;
    if (i >= nc) key = ~0ull;
    else if (i == nc - 1) key = 0ull;
    else key = chunk_key(cs[c0 + i], i);
    keys[i] = key;
  }
  if (tid == 0) found = INT_MAX;
  __syncthreads();
  for (int k = 2; k <= p2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < p2; i += kSelThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t a = keys[i], c = keys[ixj];
          const bool up = (i & k) == 0;
          if ((a > c) == up) {
            keys[i] = c;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  const double final_score = (double)cs[c0 + nc - 1];
  int cnt;
  if (mode == SP_SELECT_TOP_P) {
    cnt = budget.kc[b];
  } else {
    const int per = (nc + kSelThreads - 1) / kSelThreads;
    const int a0 = min(nc, tid * per), a1 = min(nc, a0 + per);
    double s = 0.0;
    for (int pos = a0; pos < a1; ++pos) s += pos == 0 ? final_score : (double)key_score(keys[pos]);
    part[tid] = s;
    __syncthreads();
    for (int off = 1; off < kSelThreads; off <<= 1) {
      const double v = tid >= off ? part[tid - off] : 0.0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    const double target = param * part[kSelThreads - 1];
    double cum = tid > 0 ? part[tid - 1] : 0.0;
    for (int pos = a0; pos < a1; ++pos) {
      cum += pos == 0 ? final_score : (double)key_score(keys[pos]);
      if (cum >= target) {
        atomicMin(&found, pos);
        break;
      }
    }
    __syncthreads();
    cnt = found == INT_MAX ? nc : found + 1;
  }
  for (int i = tid; i < nc; i += kSelThreads) keep[c0 + i] = 0;
  __syncthreads();
  for (int pos = tid; pos < cnt; pos += kSelThreads) {
    const int idx = pos == 0 ? nc - 1 : (int)(unsigned)(keys[pos] & 0xffffffffu) - 1;
    keep[c0 + idx] = 1;
  }
  if (tid == 0) n_kept[b] = cnt;
}

}  // namespace

hipError_t launch_select(int mode, double param, const SegTable &chunks, const SelectBudget &kc,
                         int max_nc, const float *chunk_scores, uint8_t *keep, int32_t *n_kept,
                         hipStream_t st) {
  int p2 = 1;
  while (p2 < max_nc) p2 <<= 1;
  const size_t lds = (size_t)p2 * sizeof(uint64_t);
  hipError_t e = hipFuncSetAttribute((const void *)k_select,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_select, dim3(chunks.B), dim3(kSelThreads), lds, st, mode, param, chunks, kc,
                     p2, chunk_scores, keep, n_kept);
  return hipGetLastError();
}

}  // namespace sp
