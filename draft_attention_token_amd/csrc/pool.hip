// Token scores and chunk scores: centred average pooling, min-max
// normalisation, structural boosts, chunk means.
//
// Method: "Speculative prefill" (llama.cpp pull request 27692), Approach
// step 3 (1-D average pooling, W = 13; contiguous chunks, C = 32);
// "SpecPrefill — Implementation Guide", v3.1 Optimizations & Bug Fixes,
// item 5 (min-max scaling to [0, 1] before boosting and selection), v3
// Improvements item 2 (first 64 tokens x1.5, last 128 x1.3), and Chunk
// Selection (a chunk's score is the mean over the tokens it holds).
//
// k_pool: one block per 1024-token block of a prompt; the block stages its
//   tokens plus a halo of (W-1)/2 on each side in LDS (clamped to the
//   prompt), writes the pooled values and the block's min and max.
// k_minmax: one block per prompt reduces its blocks' minima and maxima in a
//   fixed order.
// k_chunk: one thread per chunk normalises, boosts and averages its tokens.
#include "sp_internal.h"

namespace sp {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kMaxHalo = (kMaxPoolWindow - 1) / 2;

__device__ __forceinline__ void block_minmax(float &mn, float &mx, float (*sh)[kPoolThreads]) {
  const int t = threadIdx.x;
  sh[0][t] = mn;
  sh[1][t] = mx;
  __syncthreads();
  for (int w = kPoolThreads / 2; w > 0; w >>= 1) {
    if (t < w) {
      sh[0][t] = fminf(sh[0][t], sh[0][t + w]);
      sh[1][t] = fmaxf(sh[1][t], sh[1][t + w]);
    }
    __syncthreads();
  }
  mn = sh[0][0];
  mx = sh[1][0];
}

__global__ __launch_bounds__(kPoolThreads) void k_pool(PoolParams p, SegTable blocks,
                                                       const float *__restrict__ imp,
                                                       float *__restrict__ pooled,
                                                       float2 *__restrict__ block_mm) {
  __shared__ float buf[kPoolBlockTokens + 2 * kMaxHalo];
  __shared__ float red[2][kPoolThreads];
  const int blk = blockIdx.x;
  const int b = seg_of(blocks, blk);
  const int64_t base = blocks.tok_off[b];
  const int64_t N = blocks.tok_off[b + 1] - base;
  const int64_t t0 = (int64_t)(blk - blocks.unit_off[b]) * kPoolBlockTokens;
  const int64_t t1 = min(N, t0 + kPoolBlockTokens);
  const int r = (p.W - 1) / 2;
  const int64_t lo = max((int64_t)0, t0 - r), hi = min(N, t1 + r);
  for (int64_t i = threadIdx.x; i < hi - lo; i += kPoolThreads) buf[i] = imp[base + lo + i];
  __syncthreads();
  float mn = INFINITY, mx = -INFINITY;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += kPoolThreads) {
    const int64_t a = max((int64_t)0, t - r), e = min(N - 1, t + r);
    float s = 0.f;
    for (int64_t i = a; i <= e; ++i) s += buf[i - lo];
    const float v = s / (float)(e - a + 1);
    pooled[base + t] = v;
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
  block_minmax(mn, mx, red);
  if (threadIdx.x == 0) block_mm[blk] = make_float2(mn, mx);
}

__global__ __launch_bounds__(kPoolThreads) void k_minmax(SegTable blocks,
                                                         const float2 *__restrict__ block_mm,
                                                         float2 *__restrict__ prompt_mm) {
  __shared__ float red[2][kPoolThreads];
  const int b = blockIdx.x;
  float mn = INFINITY, mx = -INFINITY;
  for (int i = blocks.unit_off[b] + threadIdx.x; i < blocks.unit_off[b + 1]; i += kPoolThreads) {
    const float2 v = block_mm[i];
    mn = fminf(mn, v.x);
    mx = fmaxf(mx, v.y);
  }
  block_minmax(mn, mx, red);
  if (threadIdx.x == 0) prompt_mm[b] = make_float2(mn, mx);
}

__global__ __launch_bounds__(kPoolThreads) void k_chunk(PoolParams p, SegTable chunks,
                                                        const float *pooled,
                                                        const float2 *__restrict__ prompt_mm,
                                                        float *token_scores,
                                                        float *__restrict__ chunk_scores) {
  const int c = blockIdx.x * kPoolThreads + threadIdx.x;
  if (c >= chunks.unit_off[chunks.B]) return;
  const int b = seg_of(chunks, c);
  const int64_t base = chunks.tok_off[b];
  const int64_t N = chunks.tok_off[b + 1] - base;
  const float2 mm = prompt_mm[b];
  const float mn = mm.x, range = mm.y - mm.x;
  const bool flat = range <= 1e-6f * mm.y;
  const int64_t s0 = (int64_t)(c - chunks.unit_off[b]) * p.C, s1 = min(N, s0 + p.C);
  float sum = 0.f;
  for (int64_t t = s0; t < s1; ++t) {
    float x = pooled[base + t];
    if (p.normalize) x = flat ? 1.f : (x - mn) / range;
    if (t < p.first_n) x *= p.first_mult;
    if (t >= N - p.last_n) x *= p.last_mult;
    if (token_scores) token_scores[base + t] = x;
    sum += x;
  }
  chunk_scores[c] = sum / (float)(s1 - s0);
}

}  // namespace

size_t pool_ws(int B, int total_blocks, int64_t total_tokens) {
  return align_up((size_t)total_blocks * sizeof(float2)) + align_up((size_t)B * sizeof(float2)) +
         align_up((size_t)total_tokens * sizeof(float));
}

hipError_t launch_pool_chunk(const PoolParams &p, const SegTable &blocks, int total_blocks,
                             const SegTable &chunks, int total_chunks, const float *imp,
                             float *token_scores, float *chunk_scores, void *ws, hipStream_t st) {
  char *w = reinterpret_cast<char *>(ws);
  float2 *block_mm = reinterpret_cast<float2 *>(w);
  w += align_up((size_t)total_blocks * sizeof(float2));
  float2 *prompt_mm = reinterpret_cast<float2 *>(w);
  w += align_up((size_t)blocks.B * sizeof(float2));
  float *pooled = token_scores ? token_scores : reinterpret_cast<float *>(w);
  hipLaunchKernelGGL(k_pool, dim3(total_blocks), dim3(kPoolThreads), 0, st, p, blocks, imp, pooled,
                     block_mm);
  hipLaunchKernelGGL(k_minmax, dim3(blocks.B), dim3(kPoolThreads), 0, st, blocks, block_mm,
                     prompt_mm);
  hipLaunchKernelGGL(k_chunk, dim3((total_chunks + kPoolThreads - 1) / kPoolThreads),
                     dim3(kPoolThreads), 0, st, p, chunks, pooled, prompt_mm, token_scores,
                     chunk_scores);
  return hipGetLastError();
}

}  // namespace sp
