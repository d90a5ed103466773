// Chunk selection: fixed top-p or cumulative attention mass, per prompt.
//
// Method: "Speculative prefill" (llama.cpp pull request 27692), Approach
// step 4 (keep the top-p fraction of chunks plus BOS and the prompt
// boundary); "SpecPrefill — Implementation Guide", v3 Improvements item 1
// (sort chunks by score and keep them from the highest down until the kept
// share of the total attention mass reaches the threshold).
//
// The final chunk is always kept. The other chunks are visited by score,
// highest first, equal scores by lower index: top-p keeps the first kc - 1
// of them; mass mode keeps a chunk while the kept sum before it (final chunk
// included) is below mass * total, so the chunk that reaches the threshold
// is kept too.
//
// No sort. A chunk's place in that order is the number of chunks ahead of
// it, and the mass walk only needs the sum of their scores, so both modes
// reduce to: for every chunk, count and sum the chunks that precede it.
// k_select computes these all-pairs counts and sums, 16 chunks per block
// with 64 lane groups splitting the other chunks, and decides each chunk
// from them; the block holding the last kept chunk writes the count. Scores
// enter as 64-bit fixed point with a scale set by the prompt's largest score
// (values below 2^48, so at most 2^14 of them sum below 2^62): every sum is
// exact integer arithmetic, independent of the order of the additions, and
// the sum ahead of a chunk grows along the order. The order compares the
// top 32 bits of the fixed-point value (two scores closer than 2^-32 of the
// largest tie and go by index; both then sit at the selection boundary),
// as one 64-bit key with the chunk index below them.
#include "sp_internal.h"

namespace sp {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kRankTile = 16;                   // chunks per block
constexpr int kGroups = kThreads / kRankTile;   // lane groups splitting the other chunks (64)
constexpr int kStage = 4096;                    // chunks staged in LDS at a time
constexpr int kPerThread = SP_MAX_CHUNKS_PER_PROMPT / kThreads;   // scores held per thread

__device__ __forceinline__ int table_prompt(const int32_t *off, int B, int u) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <bool kMass>
__global__ __launch_bounds__(kThreads) void k_select(SelectTable t, double param,
                                                     const float *__restrict__ cs,
                                                     uint8_t *__restrict__ keep,
                                                     int32_t *__restrict__ n_kept) {
  __shared__ __align__(16) unsigned long long skey[kStage];
  __shared__ __align__(16) long long sfx[kMass ? kStage : 2];
  __shared__ uint32_t rc[kWaves][kRankTile];
  __shared__ long long rs[kWaves][kRankTile];
  __shared__ float redf[kWaves];
  __shared__ long long redl[kWaves];
  const int b = table_prompt(t.blk_off, t.B, blockIdx.x);
  const int tile = blockIdx.x - t.blk_off[b];
  const int c0 = t.chunk_off[b], nc = t.chunk_off[b + 1] - c0, last = nc - 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // The prompt's scores, read once: chunk tid + kThreads * e in sc[e]; with
  // them (one round trip) the final chunk's and the lane's own chunk's.
  float sc[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int j = tid + kThreads * e;
    sc[e] = j < nc ? cs[c0 + j] : 0.f;
  }
  const int i = tile * kRankTile + (lane & (kRankTile - 1));
  const bool mine = i < last;
  const float c_last = cs[c0 + last];
  const float c_i = mine ? cs[c0 + i] : 0.f;
  // The prompt's scale, and for mass mode the fixed-point sum the chunks
  // ahead of a kept one must stay below: ceil(mass * total) - final.
  float mx = 0.f;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) mx = fmaxf(mx, sc[e]);
  mx = block_max<kWaves>(mx, redf);
  const int shift = fixed_shift(mx);
  long long need;
  if (kMass) {
    long long tot = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) tot += to_fixed(sc[e], shift);
    tot = block_sum<kWaves>(tot, redl);
    need = (long long)ceil(param * (double)tot) - to_fixed(c_last, shift);
  } else {
    need = t.kc[b] - 1;   // chunks ahead of a kept one
  }

  const int grp = wave * (64 / kRankTile) + (lane / kRankTile);
  const long long fxi = mine ? to_fixed(c_i, shift) : 0ll;
  // The order as one 64-bit key: score key on top, chunk index below, so
  // "ahead of i" is a single unsigned comparison (equal scores by index).
  const unsigned long long ki = ((unsigned long long)order_key(fxi) << 32) | (uint32_t)i;
  uint32_t n = 0;
  long long sum = 0;
  // Every chunk except the final one, in LDS-sized stages; lane group g
  // takes the g-th of kGroups equal slices of each stage (multiples of 4).
  for (int j0 = 0; j0 < last; j0 += kStage) {
    const int len = min(kStage, last - j0);
    __syncthreads();
    // Stage j0 / kThreads .. + kStage / kThreads of the register copy.
#pragma unroll
    for (int e = 0; e < kStage / kThreads; ++e) {
      const int j = tid + kThreads * e;              // within the stage
      const int ej = j0 / kThreads + e;              // register slot
      float v = 0.f;
#pragma unroll
      for (int r = 0; r < kPerThread; ++r) v = r == ej ? sc[r] : v;
      const bool in = j < len;
      const long long fx = in ? to_fixed(v, shift) : 0ll;
      skey[j] = in ? ((unsigned long long)order_key(fx) << 32) | (uint32_t)(j0 + j)
                   : ~0ull;   // padding is never ahead
      if (kMass) sfx[j] = fx;
    }
    __syncthreads();
    const int per = (len + 4 * kGroups - 1) / (4 * kGroups) * 4;
    const int a = grp * per;
    for (int j = a; j < a + per; j += 4) {
      const ulonglong2 k01 = *reinterpret_cast<const ulonglong2 *>(&skey[j]);
      const ulonglong2 k23 = *reinterpret_cast<const ulonglong2 *>(&skey[j + 2]);
      const unsigned long long kk[4] = {k01.x, k01.y, k23.x, k23.y};
      long long f[4] = {0, 0, 0, 0};
      if (kMass) {
        const longlong2 f01 = *reinterpret_cast<const longlong2 *>(&sfx[j]);
        const longlong2 f23 = *reinterpret_cast<const longlong2 *>(&sfx[j + 2]);
        f[0] = f01.x; f[1] = f01.y; f[2] = f23.x; f[3] = f23.y;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ahead = kk[u] < ki;
        n += ahead ? 1u : 0u;
        if (kMass) sum += ahead ? f[u] : 0ll;
      }
    }
  }
  // Sum over the lane groups: the 4 of a wave by shuffles, the waves in LDS.
  for (int off = kRankTile; off < 64; off <<= 1) {
    n += __shfl_xor(n, off, 64);
    if (kMass) sum += __shfl_xor(sum, off, 64);
  }
  if (lane < kRankTile) {
    rc[wave][lane] = n;
    rs[wave][lane] = sum;
  }
  __syncthreads();
  if (wave != 0 || lane >= kRankTile) return;
  n = 0;
  sum = 0;
  for (int w = 0; w < kWaves; ++w) {
    n += rc[w][lane];
    sum += rs[w][lane];
  }
  if (i > last) return;
  bool k;
  if (i == last) {
    k = true;
  } else if (kMass) {
    k = sum < need;
    // The last kept chunk (the next one in the order, with sum + fxi ahead
    // of it, is not kept) writes the count; with none kept, the first one.
    if (k && (sum + fxi >= need || (int)n == last - 1)) n_kept[b] = (int)n + 2;
    if (!k && n == 0) n_kept[b] = 1;
  } else {
    k = (long long)n < need;
  }
  keep[c0 + i] = k ? 1 : 0;
  if (tile == 0 && lane == 0 && (!kMass || last == 0)) n_kept[b] = kMass ? 1 : t.kc[b];
}

}  // namespace

int select_rank_blocks(int nc) { return (nc + kRankTile - 1) / kRankTile; }

hipError_t launch_select(int mode, double param, const SelectTable &t, const float *chunk_scores,
                         uint8_t *keep, int32_t *n_kept, hipStream_t st) {
  if (mode == SP_SELECT_MASS)
    hipLaunchKernelGGL(k_select<true>, dim3(t.blk_off[t.B]), dim3(kThreads), 0, st, t, param,
                       chunk_scores, keep, n_kept);
  else
    hipLaunchKernelGGL(k_select<false>, dim3(t.blk_off[t.B]), dim3(kThreads), 0, st, t, param,
                       chunk_scores, keep, n_kept);
  return hipGetLastError();
}

}  // namespace sp
