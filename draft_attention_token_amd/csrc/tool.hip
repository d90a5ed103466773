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
// k_legacy_rank: one thread per chunk; a chunk is in when fewer than kc
//   chunk means of its prompt are strictly larger (the same set as "reaches
//   the kc-th largest mean", ties included), counted over LDS stages.
// k_legacy_list<false>, then <true>: one block per prompt, three sweeps over
//   the prompt's tokens with block scans. A token is kept when its chunk is
//   in, when it is one of the first four or last two tokens, or when it is
//   among the first F remaining tokens in index order (F tops the count up to
//   the effective minimum). The first launch stores each prompt's count
//   after the cap; the second packs the prompts by those counts and writes
//   ids and positions, keeping every step-th token and the final one when the
//   count exceeds the cap.
#include "sp_internal.h"

namespace sp {
namespace {

constexpr int kStitchThreads = 256;
constexpr int kRankThreads = 256;
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
  const int b = table_prompt(t.blk_off, t.B, blockIdx.x);
  const int c0 = t.chunk_off[b], nc = t.chunk_off[b + 1] - c0;
  const int i = (blockIdx.x - t.blk_off[b]) * kRankThreads + threadIdx.x;
  const float mine = i < nc ? cs[c0 + i] : 0.f;
  int above = 0;
  for (int j0 = 0; j0 < nc; j0 += kRankStage) {
    const int len = min(kRankStage, nc - j0);
    __syncthreads();
    for (int j = threadIdx.x; j < len; j += kRankThreads) stage[j] = cs[c0 + j0 + j];
    __syncthreads();
    for (int j = 0; j < len; ++j) above += stage[j] > mine ? 1 : 0;
  }
  if (i < nc) in[c0 + i] = above < t.kc[b] ? 1 : 0;
}

// Exclusive scan of v over the block; *total gets the block's sum.
__device__ __forceinline__ int block_scan(int v, int *total, int *wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = incl - v, tot = 0;
  for (int w = 0; w < kListThreads / 64; ++w) {
    before += w < wave ? wave_tot[w] : 0;
    tot += wave_tot[w];
  }
  __syncthreads();
  *total = tot;
  return before;
}

template <bool kWrite>
__global__ __launch_bounds__(kListThreads) void k_legacy_list(
    LegacyTable t, const uint8_t *__restrict__ in, const int32_t *__restrict__ ids,
    int32_t *__restrict__ counts, int32_t *__restrict__ kept_ids, int32_t *__restrict__ kept_pos,
    int64_t *__restrict__ kept_offsets) {
  __shared__ int wave_tot[kListThreads / 64];
  __shared__ int64_t base_off;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int n = t.tok_off[b + 1] - t.tok_off[b], c0 = t.chunk_off[b], C = t.C;
  const int per = (n + kListThreads - 1) / kListThreads;
  const int t0 = min(n, tid * per), t1 = min(n, t0 + per);
  auto base = [&](int x) {
    return in[c0 + x / C] != 0 || x < 4 || (n > 4 && x >= n - 2);
  };
  // Sweep 1: chunk, first-four and last-two tokens.
  int nb = 0;
  for (int x = t0; x < t1; ++x) nb += base(x) ? 1 : 0;
  int k0;
  const int base_before = block_scan(nb, &k0, wave_tot);
  const int fill = max(0, t.eff_min[b] - k0);
  // Sweep 2: the fill takes the first `fill` other tokens in index order (a
  // token's rank among them is x minus the base tokens before it).
  int nf = 0, bcount = base_before;
  for (int x = t0; x < t1; ++x) {
    const bool bs = base(x);
    nf += (bs || x - bcount < fill) ? 1 : 0;
    bcount += bs ? 1 : 0;
  }
  int K;
  const int kept_before = block_scan(nf, &K, wave_tot);
  if (!kWrite) {
    if (tid == 0) counts[b] = min(K, t.max_keep);
    return;
  }
  if (tid == 0) {
    int64_t s = 0;
    for (int p = 0; p < b; ++p) s += counts[p];
    base_off = s;
    kept_offsets[b] = s;
    if (b == t.B - 1) {
      kept_offsets[0] = 0;
      kept_offsets[t.B] = s + counts[b];
    }
  }
  __syncthreads();
  const int64_t off = base_off;
  // Sweep 3: write, thinned to max_keep (every step-th kept token, the last
  // slot taking the final kept token) when there are more.
  const bool thin = K > t.max_keep;
  const int step = thin ? K / t.max_keep : 1;
  int ki = kept_before;
  bcount = base_before;
  for (int x = t0; x < t1; ++x) {
    const bool bs = base(x);
    const bool f = bs || x - bcount < fill;
    bcount += bs ? 1 : 0;
    if (!f) continue;
    int slot = ki;
    if (thin) {
      if (ki == K - 1) slot = t.max_keep - 1;
      else if (ki % step == 0 && ki / step < t.max_keep - 1) slot = ki / step;
      else slot = -1;
    }
    if (slot >= 0) {
      kept_ids[off + slot] = ids[t.tok_off[b] + x];
      kept_pos[off + slot] = x;
    }
    ++ki;
  }
}

}  // namespace

int legacy_rank_blocks(int nc) { return (nc + kRankThreads - 1) / kRankThreads; }

hipError_t launch_stitch(const StitchTable &t, int32_t n, const float *win_imp, float *out,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_stitch, dim3((n + kStitchThreads - 1) / kStitchThreads),
                     dim3(kStitchThreads), 0, st, t, n, win_imp, out);
  return hipGetLastError();
}

hipError_t launch_legacy(const LegacyTable &t, const float *chunk_scores, const int32_t *ids,
                         uint8_t *in, int32_t *counts, int32_t *kept_ids, int32_t *kept_pos,
                         int64_t *kept_offsets, hipStream_t st) {
  hipLaunchKernelGGL(k_legacy_rank, dim3(t.blk_off[t.B]), dim3(kRankThreads), 0, st, t,
                     chunk_scores, in);
  hipLaunchKernelGGL(k_legacy_list<false>, dim3(t.B), dim3(kListThreads), 0, st, t, in, ids,
                     counts, kept_ids, kept_pos, kept_offsets);
  hipLaunchKernelGGL(k_legacy_list<true>, dim3(t.B), dim3(kListThreads), 0, st, t, in, ids,
                     counts, kept_ids, kept_pos, kept_offsets);
  return hipGetLastError();
}

}  // namespace sp
