// Kept-token compaction: BOS plus every token of a kept chunk, in ascending
// order, with its token id and original position.
//
// Method: "SpecPrefill — Implementation Guide", Sparse Prefill (the target
// prefills only the kept tokens at their original position ids);
// "Speculative prefill" (llama.cpp pull request 27692), Approach step 4
// (kept chunks plus BOS).
//
// k_gather_scan: one block per prompt; an exact integer scan over the kept
//   chunks gives each chunk's first output slot and the prompt's count
//   (kept chunk tokens, plus one when BOS sits in a dropped chunk 0).
// k_gather_write: one block per 1024 tokens; every kept token's slot follows
//   from its chunk's slot, so the writes need no further scan.
// k_gather_fused (batches of at most 16384 chunks, one launch): each block
//   counts the kept chunks ahead of its own tokens from the flags itself
//   (at most 16 KB of them), adds the per-prompt corrections (a short final
//   chunk, BOS), scans its own chunks in LDS and writes.
#include "sp_internal.h"

namespace sp {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kWriteThreads = 1024;
constexpr int kFusedPerThread = 16;
constexpr int kFusedMaxChunks = kWriteThreads * kFusedPerThread;
static_assert(SP_MAX_PROMPTS <= kWriteThreads, "one thread per earlier prompt");

// Block-wide sums of three ints (all threads get them).
__device__ __forceinline__ int3 block_sum3(int a, int b, int c, int3 *red) {
  for (int off = 32; off > 0; off >>= 1) {
    a += __shfl_xor(a, off, 64);
    b += __shfl_xor(b, off, 64);
    c += __shfl_xor(c, off, 64);
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_int3(a, b, c);
  __syncthreads();
  int3 v = make_int3(0, 0, 0);
  for (int w = 0; w < kWriteThreads / 64; ++w) {
    v.x += red[w].x;
    v.y += red[w].y;
    v.z += red[w].z;
  }
  __syncthreads();
  return v;
}

__global__ __launch_bounds__(kScanThreads) void k_gather_scan(SegTable chunks, int C,
                                                              const uint8_t *__restrict__ keep,
                                                              int32_t *__restrict__ chunk_out,
                                                              int32_t *__restrict__ counts) {
  constexpr int kEPT = SP_MAX_CHUNKS_PER_PROMPT / kScanThreads;   // chunks per thread
  __shared__ int wave_tot[kScanThreads / 64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = chunks.unit_off[b], nc = chunks.unit_off[b + 1] - c0;
  const int N = chunks.tok_off[b + 1] - chunks.tok_off[b];
  // Thread tid owns chunks tid*kEPT .. tid*kEPT + kEPT - 1 (index order).
  int sz[kEPT];
  int mine = 0;
#pragma unroll
  for (int e = 0; e < kEPT; ++e) {
    const int c = tid * kEPT + e;
    sz[e] = (c < nc && keep[c0 + c]) ? min(C, N - c * C) : 0;
    mine += sz[e];
  }
  int incl = mine;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int run = incl - mine;
  for (int w = 0; w < wave; ++w) run += wave_tot[w];
#pragma unroll
  for (int e = 0; e < kEPT; ++e) {
    const int c = tid * kEPT + e;
    if (c < nc) chunk_out[c0 + c] = run;
    run += sz[e];
  }
  if (tid == kScanThreads - 1) counts[b] = run + (keep[c0] ? 0 : 1);
}

__global__ __launch_bounds__(kWriteThreads) void k_gather_write(
    SegTable chunks, SegTable blocks, int C, const uint8_t *__restrict__ keep,
    const int32_t *__restrict__ chunk_out, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ ids, int32_t *__restrict__ kept_ids,
    int32_t *__restrict__ kept_pos, int64_t *__restrict__ kept_offsets) {
  __shared__ int64_t base_s;
  const int blk = blockIdx.x, tid = threadIdx.x;
  const int b = seg_of(blocks, blk);
  if (tid < 64) {
    const int64_t o = wave_prompt_offsets(counts, blocks.B, b, blk == 0 ? kept_offsets : nullptr);
    if (tid == 0) base_s = o;
  }
  __syncthreads();
  const int64_t base = base_s;
  const int c0 = chunks.unit_off[b];
  const int64_t tok0 = blocks.tok_off[b];
  const int N = blocks.tok_off[b + 1] - blocks.tok_off[b];
  const int t0 = (blk - blocks.unit_off[b]) * kGatherBlockTokens;
  const int t1 = min(N, t0 + kGatherBlockTokens);
  const bool k0 = keep[c0] != 0;
  for (int t = t0 + tid; t < t1; t += kWriteThreads) {
    // All three reads at once (every index is valid): one round trip.
    const int c = t / C;
    const bool kc = keep[c0 + c] != 0;
    const int32_t slot = chunk_out[c0 + c];
    const int32_t id = ids[tok0 + t];
    int64_t out;
    if (t == 0 && !k0) out = base;
    else if (kc) out = base + (k0 ? 0 : 1) + slot + (t - c * C);
    else continue;
    kept_ids[out] = id;
    kept_pos[out] = t;
  }
}

__global__ __launch_bounds__(kWriteThreads) void k_gather_fused(
    SegTable chunks, SegTable blocks, int C, const uint8_t *__restrict__ keep,
    const int32_t *__restrict__ ids, int32_t *__restrict__ kept_ids,
    int32_t *__restrict__ kept_pos, int64_t *__restrict__ kept_offsets) {
  __shared__ int3 red[kWriteThreads / 64];
  __shared__ int wave_tot[kWriteThreads / 64];
  __shared__ int pre[kWriteThreads];
  const int blk = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = seg_of(blocks, blk);
  const int c0 = chunks.unit_off[b];
  const int64_t tok0 = blocks.tok_off[b];
  const int N = blocks.tok_off[b + 1] - blocks.tok_off[b];
  const int t0 = (blk - blocks.unit_off[b]) * kGatherBlockTokens;
  const int t1 = min(N, t0 + kGatherBlockTokens);
  const int ca = t0 / C, cb = (t1 - 1) / C;   // the block's chunks, within the prompt
  const int nb = cb - ca + 1;                  // <= kWriteThreads
  // This thread's chunk of the block, and its token (one each), read with
  // the flags ahead of the block in one round trip.
  const int c = ca + tid;
  const bool kc = tid < nb && keep[c0 + c] != 0;
  const int t = t0 + tid;
  const int tc = t / C;
  const bool kt = t < t1 && keep[c0 + tc] != 0;
  const int32_t id = t < t1 ? ids[tok0 + t] : 0;
  // Kept chunks before the prompt, and the prompt's before the block's: C
  // tokens each (none of them is its prompt's final chunk, except before
  // the prompt: corrected below).
  int before = 0, inside = 0;
#pragma unroll
  for (int e = 0; e < kFusedPerThread; ++e) {
    const int g = tid * kFusedPerThread + e;
    const bool k = g < c0 + ca && keep[g] != 0;
    before += (k && g < c0) ? 1 : 0;
    inside += (k && g >= c0) ? 1 : 0;
  }
  // Earlier prompts, one per thread (b <= SP_MAX_PROMPTS < kWriteThreads): a
  // kept final chunk holds its real size; a dropped chunk 0 still emits BOS.
  int corr = 0;
  if (tid < b) {
    const int cs = chunks.unit_off[tid], ce = chunks.unit_off[tid + 1];
    const int np = chunks.tok_off[tid + 1] - chunks.tok_off[tid];
    if (keep[ce - 1]) corr -= C - (np - (ce - cs - 1) * C);
    if (!keep[cs]) corr += 1;
  }
  const int3 tot = block_sum3(before, inside, corr, red);
  const bool k0 = keep[c0] != 0;
  const int64_t base_prompt = (int64_t)C * tot.x + tot.z;
  const int64_t base_blk = base_prompt + (k0 ? 0 : 1) + (int64_t)C * tot.y;
  // Exclusive scan of the kept sizes of the block's chunks.
  const int sz = kc ? min(C, N - c * C) : 0;
  int incl = sz;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int excl = incl - sz;
  for (int w = 0; w < wave; ++w) excl += wave_tot[w];
  pre[tid] = excl;
  __syncthreads();
  if (t < t1) {
    if (t == 0 && !k0) {
      kept_ids[base_prompt] = id;
      kept_pos[base_prompt] = 0;
    } else if (kt) {
      const int64_t out = base_blk + pre[tc - ca] + (t - tc * C);
      kept_ids[out] = id;
      kept_pos[out] = t;
    }
  }
  if (tid == 0 && t0 == 0) kept_offsets[b] = base_prompt;
  if (tid == nb - 1 && blk == (int)gridDim.x - 1) kept_offsets[b + 1] = base_blk + excl + sz;
}

}  // namespace

size_t gather_ws(int B, int total_chunks) {
  return align_up((size_t)total_chunks * sizeof(int32_t)) + align_up((size_t)B * sizeof(int32_t));
}

hipError_t launch_gather(const SegTable &chunks, const SegTable &blocks, int total_blocks, int C,
                         const uint8_t *keep, const int32_t *ids, int32_t *kept_ids,
                         int32_t *kept_pos, int64_t *kept_offsets, void *ws, hipStream_t st) {
  const int total_chunks = chunks.unit_off[chunks.B];
  int32_t *chunk_out = reinterpret_cast<int32_t *>(ws);
  int32_t *counts = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(ws) +
                                                align_up((size_t)total_chunks * sizeof(int32_t)));
  if (total_chunks <= kFusedMaxChunks) {
    hipLaunchKernelGGL(k_gather_fused, dim3(total_blocks), dim3(kWriteThreads), 0, st, chunks,
                       blocks, C, keep, ids, kept_ids, kept_pos, kept_offsets);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_gather_scan, dim3(chunks.B), dim3(kScanThreads), 0, st, chunks, C, keep,
                     chunk_out, counts);
  hipLaunchKernelGGL(k_gather_write, dim3(total_blocks), dim3(kWriteThreads), 0, st, chunks, blocks,
                     C, keep, chunk_out, counts, ids, kept_ids, kept_pos, kept_offsets);
  return hipGetLastError();
}

}  // namespace sp
