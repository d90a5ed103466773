// Standalone-tool semantics: sliding-window stitching, the legacy chunk rule
// and the cap on tokens sent to the target.
//
// Method: "SpecPrefill — Implementation Guide": Sliding Window (the worked
// window example), v3.1 Optimizations & Bug Fixes items 6-7 and Sliding
// Window Loop (v3.1 — fixed) for the windows; Configuration Reference
// (SP_CHUNK, SP_KEEP_PCT, SP_MAX_KEEP) and the chunk-selection and main-loop
// parts of its Full Source Code for the legacy rule and the cap.
//
// k_stitch: one thread per prompt token; it averages the scores of the
//   windows whose kept range holds the token (1.0 when none does).
// k_legacy_rank: 16 chunks per block, 16 thread groups splitting the other
//   chunks; a chunk is in when fewer than kc chunk means of its prompt are
//   strictly larger (the same set as "reaches the kc-th largest mean", ties
//   included), counted over LDS stages.
// A token is kept when its chunk is in, when it is one of the first four or
// last two tokens, or when it is among the first F remaining tokens in index
// order (F tops the count up to the effective minimum).
// k_legacy_scan: one block per prompt, chunk-level exact integer scans of the
//   kept and remaining tokens; each chunk gets its first kept index, the
//   prompt its count before the cap and after it.
// k_legacy_write: one thread per token; its kept index follows from its
//   chunk's scan values in O(1), and the cap (above max_keep tokens: every
//   step-th one, the final one in the last slot) picks its output slot.
#include "sp_internal.h"

namespace sp {
namespace {

constexpr int kStitchThreads = 256;
constexpr int kRankThreads = 256;
constexpr int kRankChunks = 16;                          // chunks per block
constexpr int kRankGroups = kRankThreads / kRankChunks;  // thread groups per chunk
constexpr int kRankStage = 4096;
constexpr int kListThreads = 1024;

__global__ __launch_bounds__(kStitchThreads) void k_stitch(StitchTable t, int32_t n,
                                                           const float *__restrict__ win_imp,
                                                           float *__restrict__ out) {
  const int32_t i = (int32_t)blockIdx.x * kStitchThreads + (int32_t)threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  int cnt = 0;
  for (int w = 0; w < t.n_windows; ++w) {
    const int32_t local = i - t.start[w];
    if (local >= 0 && local < t.keep[w]) {
      acc += win_imp[t.win_off[w] + local];
      ++cnt;
    }
  }
  out[i] = cnt ? acc / (float)cnt : 1.f;
}

__device__ __forceinline__ int table_prompt(const int32_t *off, int B, int u) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kRankThreads) void k_legacy_rank(LegacyTable t,
                                                              const float *__restrict__ cs,
                                                              uint8_t *__restrict__ in) {
  __shared__ float stage[kRankStage];
  __shared__ int part[kRankGroups][kRankChunks];
  const int b = table_prompt(t.blk_off, t.B, blockIdx.x);
  const int c0 = t.chunk_off[b], nc = t.chunk_off[b + 1] - c0;
  const int ci = threadIdx.x % kRankChunks, grp = threadIdx.x / kRankChunks;
  const int i = (blockIdx.x - t.blk_off[b]) * kRankChunks + ci;
  const float mine = i < nc ? cs[c0 + i] : 0.f;
  int above = 0;
  for (int j0 = 0; j0 < nc; j0 += kRankStage) {
    const int len = min(kRankStage, nc - j0);
    __syncthreads();
    for (int j = threadIdx.x; j < len; j += kRankThreads) stage[j] = cs[c0 + j0 + j];
    __syncthreads();
    for (int j = grp; j < len; j += kRankGroups) above += stage[j] > mine ? 1 : 0;
  }
  part[grp][ci] = above;
  __syncthreads();
  if (grp == 0) {
    for (int g = 1; g < kRankGroups; ++g) above += part[g][ci];
    if (i < nc) in[c0 + i] = above < t.kc[b] ? 1 : 0;
  }
}

// Always-kept tokens (0-3 and, for n > 4, n - 2 and n - 1; a set, so n - 2
// = 3 at n = 5 counts once) in [lo, x).
__device__ __forceinline__ int always_before(int n, int lo, int x) {
  int k = max(0, min(x, 4) - lo);
  if (n > 4) {
    k += (n - 2 >= 4 && n - 2 >= lo && n - 2 < x) ? 1 : 0;
    k += (n - 1 >= lo && n - 1 < x) ? 1 : 0;
  }
  return k;
}

// Per prompt, over its chunks (16 per thread, index order): base tokens
// (kept chunks whole, plus the always-kept tokens of the others) and the
// remaining tokens; exclusive scans of both give each chunk's first kept
// index, with the fill (the first `fill` remaining tokens in index order)
// counted in. Also the prompt's kept count before the cap, and the fill.
__global__ __launch_bounds__(kListThreads) void k_legacy_scan(LegacyTable t,
                                                              const uint8_t *__restrict__ in,
                                                              int32_t *__restrict__ kept_before,
                                                              int32_t *__restrict__ rest_before,
                                                              int32_t *__restrict__ counts,
                                                              int32_t *__restrict__ stats) {
  constexpr int kEPT = SP_MAX_CHUNKS_PER_PROMPT / kListThreads;   // chunks per thread
  __shared__ int tot_b[kListThreads / 64], tot_r[kListThreads / 64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = t.chunk_off[b], nc = t.chunk_off[b + 1] - c0;
  const int n = t.tok_off[b + 1] - t.tok_off[b], C = t.C;
  int nb[kEPT], nr[kEPT];
  int mb = 0, mr = 0;
#pragma unroll
  for (int e = 0; e < kEPT; ++e) {
    const int c = tid * kEPT + e;
    const int lo = c * C, size = c < nc ? min(C, n - lo) : 0;
    const int base = c < nc ? (in[c0 + c] ? size : always_before(n, lo, lo + size)) : 0;
    nb[e] = base;
    nr[e] = size - base;
    mb += nb[e];
    mr += nr[e];
  }
  int ib = mb, ir = mr;
  for (int off = 1; off < 64; off <<= 1) {
    const int ob = __shfl_up(ib, off, 64), orr = __shfl_up(ir, off, 64);
    if (lane >= off) { ib += ob; ir += orr; }
  }
  if (lane == 63) { tot_b[wave] = ib; tot_r[wave] = ir; }
  __syncthreads();
  int rb = ib - mb, rr = ir - mr, K0 = 0, R = 0;
  for (int w = 0; w < kListThreads / 64; ++w) {
    rb += w < wave ? tot_b[w] : 0;
    rr += w < wave ? tot_r[w] : 0;
    K0 += tot_b[w];
    R += tot_r[w];
  }
  const int fill = min(R, max(0, t.eff_min[b] - K0));
#pragma unroll
  for (int e = 0; e < kEPT; ++e) {
    const int c = tid * kEPT + e;
    if (c < nc) {
      kept_before[c0 + c] = rb + min(rr, fill);
      rest_before[c0 + c] = rr;
    }
    rb += nb[e];
    rr += nr[e];
  }
  if (tid == 0) {
    const int K = K0 + fill;
    counts[b] = min(K, t.max_keep);
    stats[2 * b] = K;
    stats[2 * b + 1] = fill;
  }
}

// One thread per token, 1024 tokens per block: the token's kept index
// follows from its chunk's scan values, then the cap picks its slot.
__global__ __launch_bounds__(kListThreads) void k_legacy_write(
    LegacyTable t, const uint8_t *__restrict__ in, const int32_t *__restrict__ kept_before,
    const int32_t *__restrict__ rest_before, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ stats, const int32_t *__restrict__ ids,
    int32_t *__restrict__ kept_ids, int32_t *__restrict__ kept_pos,
    int64_t *__restrict__ kept_offsets) {
  __shared__ int64_t s_off;
  const int b = table_prompt(t.wblk_off, t.B, blockIdx.x);
  const int n = t.tok_off[b + 1] - t.tok_off[b], C = t.C, c0 = t.chunk_off[b];
  const int x = (blockIdx.x - t.wblk_off[b]) * kListThreads + threadIdx.x;
  if (threadIdx.x < 64) {
    const int64_t s = wave_prompt_offsets(counts, t.B, b, nullptr);
    if (threadIdx.x == 0) {
      s_off = s;
      if (blockIdx.x == t.wblk_off[b]) {
        kept_offsets[b] = s;
        if (b == t.B - 1) kept_offsets[t.B] = s + counts[b];
      }
    }
  }
  __syncthreads();
  if (x >= n) return;
  const int c = x / C, lo = c * C;
  const int K = stats[2 * b], fill = stats[2 * b + 1];
  bool kept;
  int ki;
  if (in[c0 + c]) {
    kept = true;
    ki = kept_before[c0 + c] + (x - lo);
  } else {
    // Before x in this chunk: a always-kept tokens and x - lo - a others,
    // of which those with a rank below `fill` are kept.
    const int a = always_before(n, lo, x);
    const int rest_rank = rest_before[c0 + c] + (x - lo - a);
    const bool always = x < 4 || (n > 4 && x >= n - 2);
    kept = always || rest_rank < fill;
    ki = kept_before[c0 + c] + a + max(0, min(fill, rest_rank) - min(fill, rest_before[c0 + c]));
  }
  if (!kept) return;
  int slot = ki;
  if (K > t.max_keep) {
    const int step = K / t.max_keep;
    if (ki == K - 1) slot = t.max_keep - 1;
    else if (ki % step == 0 && ki / step < t.max_keep - 1) slot = ki / step;
    else slot = -1;
  }
  if (slot >= 0) {
    kept_ids[s_off + slot] = ids[t.tok_off[b] + x];
    kept_pos[s_off + slot] = x;
  }
}

}  // namespace

int legacy_rank_blocks(int nc) { return (nc + kRankChunks - 1) / kRankChunks; }

hipError_t launch_stitch(const StitchTable &t, int32_t n, const float *win_imp, float *out,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_stitch, dim3((n + kStitchThreads - 1) / kStitchThreads),
                     dim3(kStitchThreads), 0, st, t, n, win_imp, out);
  return hipGetLastError();
}

hipError_t launch_legacy(const LegacyTable &t, const float *chunk_scores, const int32_t *ids,
                         void *ws, int32_t *kept_ids, int32_t *kept_pos, int64_t *kept_offsets,
                         hipStream_t st) {
  const LegacyWs w = legacy_ws(t.B, t.chunk_off[t.B], ws);
  hipLaunchKernelGGL(k_legacy_rank, dim3(t.blk_off[t.B]), dim3(kRankThreads), 0, st, t,
                     chunk_scores, w.in);
  hipLaunchKernelGGL(k_legacy_scan, dim3(t.B), dim3(kListThreads), 0, st, t, w.in, w.kept_before,
                     w.rest_before, w.counts, w.stats);
  hipLaunchKernelGGL(k_legacy_write, dim3(t.wblk_off[t.B]), dim3(kListThreads), 0, st, t, w.in,
                     w.kept_before, w.rest_before, w.counts, w.stats, ids, kept_ids, kept_pos,
                     kept_offsets);
  return hipGetLastError();
}

int legacy_write_blocks(int n) { return (n + kListThreads - 1) / kListThreads; }

LegacyWs legacy_ws(int B, int total_chunks, void *base) {
  // Offsets first, as integers; pointers only from a real base (a null base
  // asks for the size alone).
  size_t off[6];
  off[0] = 0;
  off[1] = off[0] + align_up((size_t)total_chunks);
  off[2] = off[1] + align_up(sizeof(int32_t) * (size_t)total_chunks);
  off[3] = off[2] + align_up(sizeof(int32_t) * (size_t)total_chunks);
  off[4] = off[3] + align_up(sizeof(int32_t) * (size_t)B);
  off[5] = off[4] + align_up(2 * sizeof(int32_t) * (size_t)B);
  LegacyWs w = {};
  w.bytes = off[5];
  if (base) {
    char *p = reinterpret_cast<char *>(base);
    w.in = reinterpret_cast<uint8_t *>(p + off[0]);
    w.kept_before = reinterpret_cast<int32_t *>(p + off[1]);
    w.rest_before = reinterpret_cast<int32_t *>(p + off[2]);
    w.counts = reinterpret_cast<int32_t *>(p + off[3]);
    w.stats = reinterpret_cast<int32_t *>(p + off[4]);
  }
  return w;
}

}  // namespace sp
