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
// Work is split into blocks of whole chunks, TB = C * max(1, floor(256 / C))
// <= 1024 tokens of one prompt (one token per thread for C <= 256). A block
// stages its importance values plus a halo of (W-1)/2 on each side (clamped
// to the prompt) in LDS and pools them there.
// k_pool_stats: each block's min and max of the pooled values (only when
//   normalising: the scale needs the prompt's min and max).
// k_pool_minmax: per prompt, when a prompt has too many blocks for every
//   block to reduce them itself.
// k_pool_finish: pools again (cheaper than a round trip of the pooled values
//   through memory), normalises, boosts and writes the token scores, and
//   writes each chunk's mean of them as chunk_score() forms it: from the
//   chunk's boosted pooled values relative to the block's min, so that a
//   launch that does not know the prompt's min and max yet can form the
//   same sums.
#include <algorithm>

#include "sp_internal.h"

namespace sp {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kMaxHalo = (kMaxPoolWindow - 1) / 2;
constexpr int kMaxTB = 1024;
constexpr int kTargetTB = 256;
// Prompts with more blocks than this get their min and max reduced once
// (k_pool_minmax) instead of by every block of k_pool_finish.
constexpr int kFinishReduceMax = 2048;

struct BlockSpan {
  int b;           // prompt
  int64_t base;    // global offset of the prompt's token 0
  int N;           // prompt tokens
  int t0, t1;      // the block's tokens [t0, t1) within the prompt
};

__device__ __forceinline__ BlockSpan block_span(const PoolTable &pt, int blk, int TB) {
  int lo = 0, hi = pt.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pt.blk_off[mid] <= blk) lo = mid; else hi = mid - 1;
  }
  BlockSpan s;
  s.b = lo;
  s.base = pt.tok_off[s.b];
  s.N = pt.tok_off[s.b + 1] - pt.tok_off[s.b];
  s.t0 = (blk - pt.blk_off[s.b]) * TB;
  s.t1 = min(s.N, s.t0 + TB);
  return s;
}

// Pooled values of the block's tokens into out[0 .. t1 - t0) (LDS), from the
// halo-extended importance staged in buf.
__device__ __forceinline__ void pool_block(const PoolParams &p, const BlockSpan &s,
                                           const float *__restrict__ imp, float *buf, float *out) {
  const int r = (p.W - 1) / 2;
  const int lo = max(0, s.t0 - r), hi = min(s.N, s.t1 + r);
  for (int i = threadIdx.x; i < hi - lo; i += kPoolThreads) buf[i] = imp[s.base + lo + i];
  __syncthreads();
  if (r == kDefaultPoolRadius) {
    for (int t = s.t0 + threadIdx.x; t < s.t1; t += kPoolThreads)
      out[t - s.t0] = window_mean<kDefaultPoolRadius>(buf, lo, s.N, t, r);
  } else {
    for (int t = s.t0 + threadIdx.x; t < s.t1; t += kPoolThreads)
      out[t - s.t0] = window_mean<-1>(buf, lo, s.N, t, r);
  }
  __syncthreads();
}

__device__ __forceinline__ float2 block_minmax(float mn, float mx, float2 *red) {
  return sp::block_minmax<kPoolThreads / 64>(mn, mx, red);
}

__global__ __launch_bounds__(kPoolThreads) void k_pool_stats(PoolParams p, PoolTable blocks, int TB,
                                                             const float *__restrict__ imp,
                                                             float2 *__restrict__ block_mm) {
  __shared__ float buf[kMaxTB + 2 * kMaxHalo];
  __shared__ float pooled[kMaxTB];
  __shared__ float2 red[kPoolThreads / 64];
  const BlockSpan s = block_span(blocks, blockIdx.x, TB);
  pool_block(p, s, imp, buf, pooled);
  float mn = INFINITY, mx = -INFINITY;
  for (int i = threadIdx.x; i < s.t1 - s.t0; i += kPoolThreads) {
    mn = fminf(mn, pooled[i]);
    mx = fmaxf(mx, pooled[i]);
  }
  const float2 v = block_minmax(mn, mx, red);
  if (threadIdx.x == 0) block_mm[blockIdx.x] = v;
}

__global__ __launch_bounds__(kPoolThreads) void k_pool_minmax(PoolTable blocks,
                                                              const float2 *__restrict__ block_mm,
                                                              float2 *__restrict__ prompt_mm) {
  __shared__ float2 red[kPoolThreads / 64];
  const int b = blockIdx.x;
  float mn = INFINITY, mx = -INFINITY;
  for (int i = blocks.blk_off[b] + threadIdx.x; i < blocks.blk_off[b + 1]; i += kPoolThreads) {
    const float2 v = block_mm[i];
    mn = fminf(mn, v.x);
    mx = fmaxf(mx, v.y);
  }
  const float2 v = block_minmax(mn, mx, red);
  if (threadIdx.x == 0) prompt_mm[b] = v;
}

// prompt_mm: per-prompt (min, max), or null to reduce the prompt's block
// entries here (few blocks per prompt).
__global__ __launch_bounds__(kPoolThreads) void k_pool_finish(
    PoolParams p, PoolTable blocks, int TB, const float *__restrict__ imp,
    const float2 *__restrict__ block_mm, const float2 *__restrict__ prompt_mm,
    float *__restrict__ token_scores, float *__restrict__ chunk_scores) {
  __shared__ float buf[kMaxTB + 2 * kMaxHalo];
  __shared__ float xs[kMaxTB];
  __shared__ float2 red[kPoolThreads / 64];
  const BlockSpan s = block_span(blocks, blockIdx.x, TB);
  float mn = 0.f, range = 1.f;
  bool flat = false;
  if (p.normalize) {
    float2 v;
    if (prompt_mm) {
      v = prompt_mm[s.b];
    } else {
      float lo = INFINITY, hi = -INFINITY;
      for (int i = blocks.blk_off[s.b] + threadIdx.x; i < blocks.blk_off[s.b + 1];
           i += kPoolThreads) {
        const float2 w = block_mm[i];
        lo = fminf(lo, w.x);
        hi = fmaxf(hi, w.y);
      }
      v = block_minmax(lo, hi, red);
    }
    mn = v.x;
    range = v.y - v.x;
    flat = range <= 1e-6f * v.y;   // no signal: every score becomes 1
  }
  pool_block(p, s, imp, buf, xs);
  // The block's chunks (it starts on a chunk boundary of its prompt; the
  // block is the chunks' pool group, its min g from k_pool_stats or, without
  // normalisation, reduced here).
  float g;
  if (p.normalize) {
    g = block_mm[blockIdx.x].x;
  } else {
    float lo = INFINITY;
    for (int i = threadIdx.x; i < s.t1 - s.t0; i += kPoolThreads) lo = fminf(lo, xs[i]);
    g = block_minmax(lo, -INFINITY, red).x;
  }
  const int nchunk = (s.t1 - s.t0 + p.C - 1) / p.C;
  for (int c = threadIdx.x; c < nchunk; c += kPoolThreads) {
    const int a = s.t0 + c * p.C, e = min(s.t1, a + p.C);
    const float rel = chunk_rel(p, s.N, xs, s.t0, a, e, g);
    chunk_scores[blocks.chunk_off[s.b] + a / p.C] =
        chunk_score(rel, boost_sum(p, s.N, a, e), g, e - a, p.normalize, flat, mn, range);
  }
  for (int t = s.t0 + threadIdx.x; t < s.t1; t += kPoolThreads) {
    float x = xs[t - s.t0];
    if (p.normalize) x = flat ? 1.f : (x - mn) / range;
    if (token_scores) token_scores[s.base + t] = boosted(p, s.N, t, x);
  }
}

}  // namespace

int pool_block_tokens(int C) { return C * std::max(1, kTargetTB / C); }

size_t pool_ws(int B, int total_blocks) {
  return align_up((size_t)total_blocks * sizeof(float2)) + align_up((size_t)B * sizeof(float2));
}

hipError_t launch_pool_chunk(const PoolParams &p, const PoolTable &blocks, const float *imp,
                             float *token_scores, float *chunk_scores, void *ws, hipStream_t st) {
  const int TB = pool_block_tokens(p.C);
  const int total_blocks = blocks.blk_off[blocks.B];
  float2 *block_mm = reinterpret_cast<float2 *>(ws);
  float2 *prompt_mm = reinterpret_cast<float2 *>(reinterpret_cast<char *>(ws) +
                                                 align_up((size_t)total_blocks * sizeof(float2)));
  const float2 *mm_arg = nullptr;
  if (p.normalize) {
    hipLaunchKernelGGL(k_pool_stats, dim3(total_blocks), dim3(kPoolThreads), 0, st, p, blocks, TB,
                       imp, block_mm);
    int most = 0;
    for (int b = 0; b < blocks.B; ++b) most = std::max(most, blocks.blk_off[b + 1] - blocks.blk_off[b]);
    if (most > kFinishReduceMax) {
      hipLaunchKernelGGL(k_pool_minmax, dim3(blocks.B), dim3(kPoolThreads), 0, st, blocks,
                         block_mm, prompt_mm);
      mm_arg = prompt_mm;
    }
  }
  hipLaunchKernelGGL(k_pool_finish, dim3(total_blocks), dim3(kPoolThreads), 0, st, p, blocks, TB,
                     imp, block_mm, mm_arg, token_scores, chunk_scores);
  return hipGetLastError();
}

}  // namespace sp
