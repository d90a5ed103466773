// Token scores, chunk scores, chunk selection and kept-token compaction of a
// batch in one launch.
//
// Method: the passages of the separate stages (pool.hip, select.hip,
// gather.hip): "Speculative prefill" (llama.cpp pull request 27692),
// Approach steps 3-4; "SpecPrefill — Implementation Guide", v3 Improvements
// items 1-2, v3.1 Optimizations & Bug Fixes item 5, Chunk Selection and
// Sparse Prefill. The results are those of the three stages, bit for bit:
// the same arithmetic in the same order, only the hand-offs differ.
//
// Why one launch: each stage needs a whole array from the one before (every
// chunk score of a prompt before any chunk is ranked, every kept count
// before any token is placed), and as separate launches each pays a launch
// and a ramp for a few microseconds of work. Here one grid of 1024-thread
// blocks, at most one per CU and all resident at once (the host checks the
// occupancy), runs the stages as phases. What crosses a phase goes through
// 64-bit workspace slots that hold the call's tag above the value, so a
// waiting block takes only values of its own call and no slot is ever
// cleared. Block g owns TB tokens of one prompt (whole chunks):
//  1. it pools its tokens (the importance halo is read from memory) and posts
//     their min and max;
//  2. it takes the prompt's min and max from its blocks' slots, normalises
//     and boosts, writes its token scores and posts its chunk scores;
//  3. it takes every chunk score of the prompt from the slots and ranks its
//     own chunks among them as sp_select_chunks does (all pairs, sums in
//     64-bit fixed point), writes their keep flags and posts its count of
//     kept tokens (BOS included in a prompt's first block);
//  4. it takes the counts of every earlier block, which place its tokens in
//     the packed output, and writes them.
// Every wait is bounded (the budget of the scoring call's waits); a block
// whose wait ends without the value records the call's tag in the
// workspace header, writes no packed output, and runs to the end, so the
// grid always drains.
#include <algorithm>
#include <mutex>

#include "sp_internal.h"

namespace sp {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kRank = 16;                    // the block's chunks ranked per pass
constexpr int kStage = 4096;                 // chunk keys staged in LDS at a time
constexpr int kPerThread = SP_MAX_CHUNKS_PER_PROMPT / kThreads;
constexpr int kHalo = (kMaxPoolWindow - 1) / 2;
constexpr int kBlockGroups = 16;             // pool groups in a block (>= 2048 / 129)
static_assert(kPostMaxChunks <= 64, "one wave scans the block's chunks");
static_assert(kPostMaxBlocks <= kThreads, "one thread per earlier block");
static_assert(kPostMaxGroups % kThreads == 0, "whole group slices per thread");

struct PostWs {
  uint32_t *hdr;     // [0]: tag of a call whose wait timed out; [1]: latest call
  uint64_t *mm;      // [groups][2]: a pool group's pooled min and max
  uint64_t *cnt;     // [kPostMaxBlocks]: a block's kept tokens
  uint64_t *cs;      // [chunks]: chunk scores
  uint32_t tag;
  uint64_t wait_ticks;
};

__device__ __forceinline__ void post(uint64_t *p, uint32_t v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The values of the slots addr(m), m < M, for which use(m), once they carry
// the call's tag; addr(m) must be a valid slot for every m (an unused one is
// read and ignored, so that every load is issued before any is waited on:
// one round trip when the values are there, and one per retry). After a
// wait that ran out (this one or an earlier one of the thread), whatever
// the slots hold.
template <int M, typename Addr, typename Use>
__device__ __forceinline__ void take(Addr addr, Use use, uint32_t (&v)[M], const PostWs &ws,
                                     bool &dead) {
  static_assert(M <= 32, "one bit per slot");
  uint64_t w[M];
#pragma unroll
  for (int m = 0; m < M; ++m)
    w[m] = __hip_atomic_load(addr(m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t missing = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    v[m] = (uint32_t)w[m];
    if (use(m) && (uint32_t)(w[m] >> 32) != ws.tag) missing |= 1u << m;
  }
  if (missing && !dead) {
    const uint64_t t0 = wall_clock64();
    do {
      if (wall_clock64() - t0 > ws.wait_ticks) {
        __hip_atomic_store(ws.hdr, ws.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        dead = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      // All of them again, in flight together (one round trip per retry).
      uint64_t x[M];
#pragma unroll
      for (int m = 0; m < M; ++m)
        x[m] = __hip_atomic_load(addr(m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (missing & (1u << m)) {
          v[m] = (uint32_t)x[m];
          if ((uint32_t)(x[m] >> 32) == ws.tag) missing &= ~(1u << m);
        }
      }
    } while (missing);
  }
}

template <bool kMass>
__global__ __launch_bounds__(kThreads) void k_post(
    PoolParams p, PostTable t, double param, const float *__restrict__ imp,
    const int32_t *__restrict__ ids, float *__restrict__ token_scores,
    float *__restrict__ chunk_scores, uint8_t *__restrict__ keep, int32_t *__restrict__ n_kept,
    int32_t *__restrict__ kept_ids, int32_t *__restrict__ kept_pos,
    int64_t *__restrict__ kept_offsets, PostWs ws) {
  __shared__ float buf[kPostMaxTB + 2 * kHalo];
  __shared__ float xs[kPostMaxTB];
  __shared__ float gmin[kPostMaxGroups];                 // the prompt's pool-group mins
  __shared__ uint32_t bmn[kBlockGroups], bmx[kBlockGroups];   // the block's groups
  // Chunk sums by runs of 8: a block's chunks hold at most kPostMaxTB tokens
  // in at most kPostMaxChunks chunks, so at most this many runs.
  __shared__ float xpart[kPostMaxTB / 8 + kPostMaxChunks];
  __shared__ __align__(16) unsigned long long skey[kStage];
  __shared__ __align__(16) long long sfx[kMass ? kStage : 2];
  __shared__ float2 redf2[kWaves];
  __shared__ float redf[kWaves];
  __shared__ long long redl[kWaves];
  __shared__ uint32_t rc[4 * kWaves][kRank];             // a pass's partials by (wave, row)
  __shared__ long long rs[kMass ? 4 * kWaves : 1][kRank];
  __shared__ uint32_t rnn[kPostMaxChunks];                 // chunks ahead of each block chunk
  __shared__ long long rss[kMass ? kPostMaxChunks : 1];   // and their fixed-point sum
  __shared__ float csb[kPostMaxChunks];   // the block's chunk scores
  __shared__ int ksz[kPostMaxChunks];     // kept tokens per chunk of the block
  __shared__ int kpre[kPostMaxChunks];    // their exclusive prefix
  __shared__ long long fx_last;           // the prompt's final chunk in fixed point
  const int g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bool dead = false;
  if (g == 0 && tid == 0) ws.hdr[1] = ws.tag;
  int b = 0;
  {
    int lo = 0, hi = t.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (t.blk_off[mid] <= g) lo = mid; else hi = mid - 1;
    }
    b = lo;
  }
  const int64_t tok0 = t.tok_off[b];
  const int N = t.tok_off[b + 1] - t.tok_off[b];
  const int t0 = (g - t.blk_off[b]) * t.TB, t1 = min(N, t0 + t.TB);
  const int c0 = t.chunk_off[b], nc = t.chunk_off[b + 1] - c0, last = nc - 1;
  const int ca = t0 / p.C, nck = (t1 - t0 + p.C - 1) / p.C;   // the block's chunks
  const int GT = t.GT;                                         // tokens per pool group
  const int q0 = t.grp_off[b], nq = t.grp_off[b + 1] - q0;     // the prompt's groups
  const int qa = t0 / GT, nqb = (t1 - t0 + GT - 1) / GT;       // the block's groups

  // 1. Pooled values of the block's tokens (as k_pool_finish), each pool
  //    group's min and max, and each chunk's boosted sum relative to its
  //    group's min; all of them posted.
  {
    const int r = (p.W - 1) / 2;
    const int lo = max(0, t0 - r), hi = min(N, t1 + r);
    for (int i = tid; i < hi - lo; i += kThreads) buf[i] = imp[tok0 + lo + i];
    if (tid < nqb) {
      bmn[tid] = ord_of(INFINITY);
      bmx[tid] = ord_of(-INFINITY);
    }
    __syncthreads();
    // (Waves do not straddle groups when GT is a multiple of 64: then one
    // lane per wave takes the wave's min and max to LDS.)
    const bool whole = GT % 64 == 0;
    for (int tt0 = t0; tt0 < t1; tt0 += kThreads) {
      const int tt = tt0 + tid;
      float x = 0.f;
      if (tt < t1) {
        x = r == kDefaultPoolRadius ? window_mean<kDefaultPoolRadius>(buf, lo, N, tt, r)
                                    : window_mean<-1>(buf, lo, N, tt, r);
        xs[tt - t0] = x;
      }
      if (whole) {
        const int wt = tt0 + wave * 64;   // the wave's first token
        if (wt < t1) {
          const float wmn = wave_min(tt < t1 ? x : INFINITY);
          const float wmx = wave_max(tt < t1 ? x : -INFINITY);
          if (lane == 0) {
            atomicMin(&bmn[(wt - t0) / GT], ord_of(wmn));
            atomicMax(&bmx[(wt - t0) / GT], ord_of(wmx));
          }
        }
      } else if (tt < t1) {
        atomicMin(&bmn[(tt - t0) / GT], ord_of(x));
        atomicMax(&bmx[(tt - t0) / GT], ord_of(x));
      }
    }
    __syncthreads();
  }
  if (tid < nqb) {
    post(ws.mm + 2 * (q0 + qa + tid), __float_as_uint(float_of(bmn[tid])), ws.tag);
    post(ws.mm + 2 * (q0 + qa + tid) + 1, __float_as_uint(float_of(bmx[tid])), ws.tag);
  }
  {
    // Each chunk's runs of 8 tokens on lanes of their own, then the partials
    // in order (as chunk_rel adds them).
    const int runs = (p.C + 7) / 8;   // per chunk
    for (int w0 = 0; w0 < nck * runs; w0 += kThreads) {
      const int k = w0 + tid, c = k / runs, u = k - c * runs;
      if (k < nck * runs) {
        const int a = t0 + c * p.C, e = min(t1, a + p.C);
        xpart[k] = a + 8 * u < e ? chunk_part(p, N, xs, t0, a + 8 * u, e, float_of(bmn[(a - t0) / GT]))
                                 : 0.f;
      }
    }
    __syncthreads();
    for (int c = tid; c < nck; c += kThreads) {
      const int a = t0 + c * p.C, e = min(t1, a + p.C);
      float rel = 0.f;
      for (int u = 0; a + 8 * u < e; ++u) rel = __fadd_rn(rel, xpart[c * runs + u]);
      post(ws.cs + c0 + ca + c, __float_as_uint(rel), ws.tag);
    }
  }

  const int ept = (nc + kThreads - 1) / kThreads;   // sc[] slots in use (uniform)

  // 2. Every group's min and max and every chunk's sum of the prompt: the
  //    prompt's min and max, every chunk score (chunk tid + kThreads * e in
  //    sc[e]), the block's token scores.
  float sc[kPerThread];
  {
    constexpr int kQ = kPostMaxGroups / kThreads;   // groups per thread
    uint32_t got[2 * kQ + kPerThread];
    take(
        [&](int m) {
          if (m < 2 * kQ) {
            const int k = tid + kThreads * (m >> 1);
            return ws.mm + 2 * (q0 + (k < nq ? k : 0)) + (m & 1);
          }
          const int j = tid + kThreads * (m - 2 * kQ);
          return ws.cs + c0 + (j < nc ? j : 0);
        },
        [&](int m) {
          return m < 2 * kQ ? tid + kThreads * (m >> 1) < nq : tid + kThreads * (m - 2 * kQ) < nc;
        },
        got, ws, dead);
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int k = tid + kThreads * q;
      if (k < nq) {
        gmin[k] = __uint_as_float(got[2 * q]);
        lo = fminf(lo, __uint_as_float(got[2 * q]));
        hi = fmaxf(hi, __uint_as_float(got[2 * q + 1]));
      }
    }
    float mn = 0.f, range = 1.f;
    bool flat = false;
    const float2 pm = block_minmax<kWaves>(lo, hi, redf2);   // also publishes gmin
    if (p.normalize) {
      mn = pm.x;
      range = pm.y - pm.x;
      flat = range <= 1e-6f * pm.y;   // no signal: every score becomes 1
    }
    for (int tt = t0 + tid; tt < t1; tt += kThreads) {
      float x = xs[tt - t0];
      if (p.normalize) x = flat ? 1.f : (x - mn) / range;
      if (token_scores) token_scores[tok0 + tt] = boosted(p, N, tt, x);
    }
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int j = tid + kThreads * e;
      sc[e] = 0.f;
      if (e < ept && j < nc) {
        const int a = j * p.C, en = min(N, a + p.C);
        sc[e] = chunk_score(__uint_as_float(got[2 * kQ + e]), boost_sum(p, N, a, en), gmin[a / GT],
                            en - a, p.normalize, flat, mn, range);
        if (j >= ca && j < ca + nck) {
          chunk_scores[c0 + j] = sc[e];
          csb[j - ca] = sc[e];
        }
      }
    }
  }

  // 3. The scale and threshold of the prompt's selection; the keys of the
  //    prompt's first kStage chunks go straight to LDS.
  float mx = 0.f;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) mx = fmaxf(mx, sc[e]);
  mx = block_max<kWaves>(mx, redf);   // syncs csb too
  const int shift = fixed_shift(mx);
  long long tot = 0;   // fixed-point sum of the thread's chunks
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    if (e < ept) {
      const int j = tid + kThreads * e;
      const long long fx = j < nc ? to_fixed(sc[e], shift) : 0ll;
      tot += fx;
      if (j == last) fx_last = fx;   // the final chunk's
      if (e < kStage / kThreads) {
        const bool in = j < last;
        skey[j] = in ? ((unsigned long long)order_key(fx) << 32) | (uint32_t)j : ~0ull;
        if (kMass) sfx[j] = in ? fx : 0ll;
      }
    }
  }
  long long need;
  if (kMass) {
    tot = block_sum<kWaves>(tot, redl);   // syncs the first stage's keys and fx_last too
    need = (long long)ceil(param * (double)tot) - fx_last;
  } else {
    need = t.kc[b] - 1;   // chunks ahead of a kept one
  }
  // For each of the block's chunks, the number (and for mass, the fixed-point
  // sum) of the prompt's non-final chunks ahead of it in the order (score key
  // above, chunk index below: an ascending key is a descending score, equal
  // scores by index), from all pairs as in sp_select_chunks. Here a group of
  // 4 lanes shares each LDS key read: lane slot s = lane & 3 holds 4 of the
  // pass's kRank chunks (s, s + 4, s + 8, s + 12) and the tid / 4-th of
  // kThreads / 4 slices of every stage of the prompt's keys.
  if (!kMass) __syncthreads();   // the first stage's keys (block_sum synced them for mass)
  const int s4 = lane & 3, gi = tid >> 2;
  const int npass = (nck + kRank - 1) / kRank;
  for (int ps = 0; ps < npass; ++ps) {
    unsigned long long ki[4];
    uint32_t n[4] = {0, 0, 0, 0};
    long long sum[4] = {0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = ps * kRank + s4 + 4 * q, i = ca + c;
      const long long fxi = (c < nck && i < last) ? to_fixed(csb[c], shift) : 0ll;
      ki[q] = ((unsigned long long)order_key(fxi) << 32) | (uint32_t)i;
    }
    for (int j0 = 0; j0 < last; j0 += kStage) {
      const int len = min(kStage, last - j0);
      if (j0 > 0 || (ps > 0 && last > kStage)) {
        // Later stages (prompts of more than kStage chunks; for a later pass,
        // every stage again) from the registers.
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kStage / kThreads; ++e) {
          const int j = tid + kThreads * e;   // within the stage
          const int ej = j0 / kThreads + e;   // register slot
          float v = 0.f;
#pragma unroll
          for (int q = 0; q < kPerThread; ++q) v = q == ej ? sc[q] : v;
          const bool in = j < len;
          const long long fx = in ? to_fixed(v, shift) : 0ll;
          skey[j] = in ? ((unsigned long long)order_key(fx) << 32) | (uint32_t)(j0 + j)
                       : ~0ull;   // padding is never ahead
          if (kMass) sfx[j] = fx;
        }
        __syncthreads();
      }
      const int per = (len + 2 * (kThreads / 4) - 1) / (2 * (kThreads / 4)) * 2;
      for (int j = gi * per; j < gi * per + per; j += 2) {
        const ulonglong2 k2 = *reinterpret_cast<const ulonglong2 *>(&skey[j]);
        longlong2 f2 = make_longlong2(0, 0);
        if (kMass) f2 = *reinterpret_cast<const longlong2 *>(&sfx[j]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool a0 = k2.x < ki[q], a1 = k2.y < ki[q];
          n[q] += (a0 ? 1u : 0u) + (a1 ? 1u : 0u);
          if (kMass) sum[q] += (a0 ? f2.x : 0ll) + (a1 ? f2.y : 0ll);
        }
      }
    }
    // Over the 16 lanes of a wave with the same slot: rotations by 4 and 8
    // within each row of 16, then the rows and waves through LDS.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#define SP_ROT_ADD(ctrl)                                                                      \
  {                                                                                           \
    n[q] += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)n[q], ctrl, 0xf, 0xf, false);       \
    if (kMass) {                                                                              \
      const uint32_t l2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)sum[q], ctrl, 0xf, 0xf, false); \
      const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp(                              \
          0, (int)(uint32_t)((unsigned long long)sum[q] >> 32), ctrl, 0xf, 0xf, false);       \
      sum[q] += (long long)(((unsigned long long)h2 << 32) | l2);                             \
    }                                                                                         \
  }
      SP_ROT_ADD(0x124) SP_ROT_ADD(0x128)
#undef SP_ROT_ADD
      if ((lane & 12) == 0) {
        rc[wave * 4 + (lane >> 4)][s4 + 4 * q] = n[q];
        if (kMass) rs[wave * 4 + (lane >> 4)][s4 + 4 * q] = sum[q];
      }
    }
    __syncthreads();
    if (tid < kRank && ps * kRank + tid < nck) {
      uint32_t nn = 0;
      long long ss = 0;
      for (int w = 0; w < 4 * kWaves; ++w) {
        nn += rc[w][tid];
        if (kMass) ss += rs[w][tid];
      }
      rnn[ps * kRank + tid] = nn;
      if (kMass) rss[ps * kRank + tid] = ss;
    }
    __syncthreads();
  }
  if (tid < nck) {
    const int c = tid, i = ca + c;
    const uint32_t nn = rnn[c];
    const long long ss = kMass ? rss[c] : 0ll;
    bool k;
    if (i == last) {
      k = true;
    } else if (kMass) {
      const long long f = to_fixed(csb[c], shift);
      k = ss < need;
      // The last kept chunk (the next one in the order, with ss + f ahead of
      // it, is not kept) writes the count; with none kept, the first one.
      if (k && (ss + f >= need || (int)nn == last - 1)) n_kept[b] = (int)nn + 2;
      if (!k && nn == 0) n_kept[b] = 1;
    } else {
      k = (long long)nn < need;
    }
    keep[c0 + i] = k ? 1 : 0;
    ksz[c] = k ? min(p.C, N - i * p.C) : 0;
  }
  if (tid == 0 && t0 == 0 && (!kMass || last == 0)) n_kept[b] = kMass ? 1 : t.kc[b];
  __syncthreads();

  // The block's kept tokens (BOS in a prompt's first block when chunk 0 is
  // dropped) and their prefix over its chunks.
  const bool bos = t0 == 0 && ksz[0] == 0;
  if (wave == 0) {
    const int v = lane < nck ? ksz[lane] : 0;
    int incl = v;
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane < nck) kpre[lane] = incl - v;
    if (lane == 63) post(ws.cnt + g, (uint32_t)(incl + (bos ? 1 : 0)), ws.tag);
  }
  // 4. The kept tokens of every earlier block place this block's.
  long long base;
  {
    uint32_t got[1];
    take([&](int) { return ws.cnt + (tid < g ? tid : 0); }, [&](int) { return tid < g; }, got, ws,
         dead);
    base = tid < g ? (long long)got[0] : 0ll;
  }
  base = block_sum<kWaves>(base, redl);   // syncs kpre
  // A wait that ran out anywhere in the block leaves its counts unknown:
  // then nothing is written at a position they would give.
  if (__syncthreads_or(dead ? 1 : 0)) return;
  const int64_t total = t.tok_off[t.B];
  if (tid == 0 && t0 == 0) kept_offsets[b] = base;
  if (bos && tid == 0 && base < total) {
    kept_ids[base] = ids[tok0];
    kept_pos[base] = 0;
  }
  const long long first = base + (bos ? 1 : 0);
  for (int tt = t0 + tid; tt < t1; tt += kThreads) {
    const int c = tt / p.C - ca;
    if (ksz[c] == 0) continue;
    const long long out = first + kpre[c] + (tt - (ca + c) * p.C);
    if (out >= total) continue;
    kept_ids[out] = ids[tok0 + tt];
    kept_pos[out] = tt;
  }
  if (tid == 0 && g == (int)gridDim.x - 1)
    kept_offsets[t.B] = first + kpre[nck - 1] + ksz[nck - 1];
}

// The header of a call that runs the separate kernels: no wait of it timed out.
__global__ void k_stamp(uint32_t *hdr, uint32_t tag) {
  hdr[0] = 0u;
  hdr[1] = tag;
}

}  // namespace

int post_max_blocks() {
  constexpr int kMaxDevices = 64;
  static int blocks[kMaxDevices];
  static bool done[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!done[dev]) {
    done[dev] = true;
    int cus = 0, a = 0, c = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, k_post<true>, kThreads, 0) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&c, k_post<false>, kThreads, 0) == hipSuccess &&
        a >= 1 && c >= 1)
      blocks[dev] = std::min(cus, kPostMaxBlocks);
  }
  return blocks[dev];
}

size_t post_slot_bytes(int total_chunks, int total_groups) {
  return align_up((size_t)total_groups * 2 * sizeof(uint64_t)) +
         align_up((size_t)kPostMaxBlocks * sizeof(uint64_t)) +
         align_up((size_t)total_chunks * sizeof(uint64_t));
}

hipError_t launch_post(int mode, double param, const PoolParams &p, const PostTable &t,
                       const float *imp, const int32_t *ids, float *token_scores,
                       float *chunk_scores, uint8_t *keep, int32_t *n_kept, int32_t *kept_ids,
                       int32_t *kept_pos, int64_t *kept_offsets, void *ws, hipStream_t st) {
  PostWs w;
  char *base = reinterpret_cast<char *>(ws);
  w.hdr = reinterpret_cast<uint32_t *>(base);
  base += kStatusBytes;
  w.mm = reinterpret_cast<uint64_t *>(base);
  base += align_up((size_t)t.grp_off[t.B] * 2 * sizeof(uint64_t));
  w.cnt = reinterpret_cast<uint64_t *>(base);
  base += align_up((size_t)kPostMaxBlocks * sizeof(uint64_t));
  w.cs = reinterpret_cast<uint64_t *>(base);
  w.tag = reserve_tags(1);
  w.wait_ticks = score_wait_ticks();
  const int grid = t.blk_off[t.B];
  if (mode == SP_SELECT_MASS)
    hipLaunchKernelGGL(k_post<true>, dim3(grid), dim3(kThreads), 0, st, p, t, param, imp, ids,
                       token_scores, chunk_scores, keep, n_kept, kept_ids, kept_pos, kept_offsets, w);
  else
    hipLaunchKernelGGL(k_post<false>, dim3(grid), dim3(kThreads), 0, st, p, t, param, imp, ids,
                       token_scores, chunk_scores, keep, n_kept, kept_ids, kept_pos, kept_offsets, w);
  return hipGetLastError();
}

hipError_t launch_stamp(void *ws, hipStream_t st) {
  hipLaunchKernelGGL(k_stamp, dim3(1), dim3(1), 0, st, reinterpret_cast<uint32_t *>(ws),
                     reserve_tags(1));
  return hipGetLastError();
}

}  // namespace sp
