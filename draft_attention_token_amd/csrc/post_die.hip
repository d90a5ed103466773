// Token scores, chunk scores, chunk selection and kept-token compaction of a
// batch in one launch whose blocks exchange values only with blocks on their
// own chip die.
//
// Method: the passages of the separate stages (pool.hip, select.hip,
// gather.hip): "Speculative prefill" (llama.cpp pull request 27692),
// Approach steps 3-4; "SpecPrefill — Implementation Guide", v3 Improvements
// items 1-2, v3.1 Optimizations & Bug Fixes item 5, Chunk Selection and
// Sparse Prefill. The results are those of the three stages, bit for bit.
//
// Why this form: a value one block stores reaches a block on another die
// (XCD) only through memory, ~1.3-1.5 us, and a waiting block sees it one
// or two polls later, so each exchange across dies costs ~5 us; a plain
// store stays in the writer's L2, where a device-scope load of a block on
// the same die finds it a fraction of a microsecond later. Here every die
// runs the whole batch, so no value has to leave a die:
//  * the batch is cut into NR ranges of TB tokens (whole pool groups of one
//    prompt); block c takes range c / 8 and runs on die c % 8 (a launch
//    deals blocks to the dies in turn; only the speed rests on that);
//  1. each block pools its range and posts its pool groups' min and max and
//     its chunks' boosted sums relative to the group min (as post.hip);
//  2. it takes every group and chunk slot of its prompt: the prompt's min
//     and max, and every chunk score;
//  3. it finds the prompt's selection cutoff itself: a radix select over
//     the chunk keys (score key above, index below) whose bins also carry
//     the fixed-point score sums, so that the mass ahead of each bin is
//     exact; every block of the prompt, on every die, gets the same cutoff;
//  4. from the cutoff it knows every chunk's keep flag, hence the kept
//     tokens ahead of each of its chunks, and writes the eighth of its range
//     that belongs to its die; for a batch of several prompts it first takes
//     the kept-token counts of the earlier prompts (posted on its die).
// Slots are 64-bit, the call's tag above a 32-bit value; each is written
// twice: a plain store (what a poll on the same die finds) and a
// device-scope store, read by every eighth poll in case a block runs on
// another die than its number says. Every wait is bounded (the scoring
// call's budget); a block whose wait ends without the value marks the call
// in the workspace header, writes no packed output and runs to the end.
#include <algorithm>
#include <mutex>

#include "sp_internal.h"

namespace sp {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
static_assert(kWaves <= 16, "one wave value per lane of a row of 16");
// Chunk scores per thread: the fewest of kMinEPT, 2 kMinEPT and kMaxEPT that
// hold the batch's largest prompt (registers are allocated for all of them).
constexpr int kMinEPT = 4096 / kThreads;
constexpr int kMaxEPT = SP_MAX_CHUNKS_PER_PROMPT / kThreads;
constexpr int kHalo = (kMaxPoolWindow - 1) / 2;
// Pool groups of a range: a group holds C * floor(256 / C) >= 129 tokens.
constexpr int kMinGroupTokens = 129;
constexpr int kRangeGroups = (kDieMaxTB + kMinGroupTokens - 1) / kMinGroupTokens;
constexpr int kBins = 256;                                        // radix digit: 8 bits
constexpr int kKeyBits = 46;                                      // 32-bit score key + 14-bit index
constexpr int kWriteMax = (kDieMaxTB + kXcds - 1) / kXcds;        // tokens a block writes
// The chunks a block writes: at most kWriteMax (one-token chunks), else at
// most kWriteMax / 2 + 2; kScanPer consecutive ones per thread in the scan.
constexpr int kScanPer = (kWriteMax + kThreads - 1) / kThreads;
static_assert(kPostMaxGroups % kThreads == 0, "whole group slices per thread");
static_assert(SP_MAX_CHUNKS_PER_PROMPT <= (1 << (kKeyBits - 32)), "chunk index below the score key");
static_assert(kDieMaxPrompts <= kThreads, "one thread per earlier prompt");

struct DieWs {
  uint32_t *hdr;        // [0]: tag of a call whose wait timed out; [1]: latest call
  uint64_t *slots;      // [2 copies][kXcds dies][per]: plain-store copy, device-scope copy
  int64_t per;          // words per (copy, die)
  int64_t cs0, cnt0;    // word offsets in a region: chunk sums, prompt counts (groups at 0)
  uint32_t tag;
  uint64_t wait_ticks;
};

__device__ __forceinline__ uint64_t *region(const DieWs &ws, int copy, int die) {
  return ws.slots + (int64_t)(copy * kXcds + die) * ws.per;
}

// Posts v at word `at` of die d's slots: a plain store, which stays in this
// die's L2, and a device-scope one.
__device__ __forceinline__ void post(const DieWs &ws, int d, int64_t at, uint32_t v) {
  const uint64_t w = ((uint64_t)ws.tag << 32) | v;
  region(ws, 0, d)[at] = w;
  __hip_atomic_store(region(ws, 1, d) + at, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t poll_load(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The values at words at(m), m < M, of die d's slots for which use(m), once
// they carry the call's tag; at(m) must be a valid word for every m (an
// unused one is read and ignored, so that every load is issued before any
// is waited on: one round trip when the values are there, and one per
// retry). Polls read the plain-store copy, every eighth the device-scope
// one. After a wait that ran out (this one or an earlier one of the
// thread), whatever the slots hold.
template <int M, typename At, typename Use>
__device__ __forceinline__ void take(At at, Use use, uint32_t (&v)[M], const DieWs &ws, int d,
                                     bool &dead) {
  static_assert(M <= 64, "one bit per slot");
  const uint64_t *near = region(ws, 0, d), *far = region(ws, 1, d);
  uint64_t w[M];
#pragma unroll
  for (int m = 0; m < M; ++m) w[m] = poll_load(near + at(m));
  uint64_t missing = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    v[m] = (uint32_t)w[m];
    if (use(m) && (uint32_t)(w[m] >> 32) != ws.tag) missing |= 1ull << m;
  }
  if (missing && !dead) {
    const uint64_t t0 = wall_clock64();
    for (int round = 1;; ++round) {
      if (wall_clock64() - t0 > ws.wait_ticks) {
        __hip_atomic_store(ws.hdr, ws.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        dead = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      const uint64_t *src = (round & 7) == 0 ? far : near;
      uint64_t x[M];
#pragma unroll
      for (int m = 0; m < M; ++m) x[m] = poll_load(src + at(m));   // all again, in flight together
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (missing & (1ull << m)) {
          v[m] = (uint32_t)x[m];
          if ((uint32_t)(x[m] >> 32) == ws.tag) missing &= ~(1ull << m);
        }
      }
      if (!missing) break;
    }
  }
}

// Inclusive scans over the wave in lane order, by DPP: shifts by 1, 2, 4
// and 8 within each row of 16 lanes, then row 0's total added to row 1 and
// row 2's to row 3 (row_bcast:15), then lane 31's to rows 2 and 3
// (row_bcast:31). Lanes without a source add 0.
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);
  return x;
}
__device__ __forceinline__ long long wave_scan_i64(long long v) {
  unsigned long long x = (unsigned long long)v;
#define SP_DPP_SCAN64(ctrl, rm)                                                                 \
  {                                                                                             \
    const uint32_t l2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, ctrl, rm, 0xf, false); \
    const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), ctrl, rm, 0xf, false); \
    x += ((unsigned long long)h2 << 32) | l2;                                                   \
  }
  SP_DPP_SCAN64(0x111, 0xf) SP_DPP_SCAN64(0x112, 0xf) SP_DPP_SCAN64(0x114, 0xf)
  SP_DPP_SCAN64(0x118, 0xf) SP_DPP_SCAN64(0x142, 0xa) SP_DPP_SCAN64(0x143, 0xc)
#undef SP_DPP_SCAN64
  return (long long)x;
}

// A chunk's radix key: the score key above its index (both ascending: the
// higher score first, equal scores by index).
__device__ __forceinline__ unsigned long long chunk_key(long long fx, int j) {
  return ((unsigned long long)order_key(fx) << (kKeyBits - 32)) | (unsigned long long)j;
}

// State of the radix select, shared through LDS: candidates are the keys k
// with k >> top == P; this pass's digit is bits [sh, top). bc / bm: count
// and fixed-point sum of the keys below every candidate.
struct SelState {
  unsigned long long P;
  long long bm;
  int bc, sh, top, done;
};

// x moved across lanes by a DPP control (4- or 8-byte types).
template <int kCtrl, typename T>
__device__ __forceinline__ T dpp_mov(T x) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(
        T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, false));
  } else {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
    const uint32_t l = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, kCtrl, 0xf, 0xf, false);
    const uint32_t h =
        (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), kCtrl, 0xf, 0xf, false);
    return __builtin_bit_cast(T, ((unsigned long long)h << 32) | l);
  }
}
// op over each row of 16 lanes, in every lane of the row.
template <typename T, typename Op>
__device__ __forceinline__ T row_fold(T x, Op op) {
  x = op(x, dpp_mov<0xB1>(x));    // lane ^ 1
  x = op(x, dpp_mov<0x4E>(x));    // lane ^ 2
  x = op(x, dpp_mov<0x124>(x));   // rotate the row by 4
  x = op(x, dpp_mov<0x128>(x));   // and by 8
  return x;
}
// The waves' values red[0 .. kWaves) folded with op, in every lane: one LDS
// read per lane (id, the identity of op, past kWaves), a row fold.
template <typename T, typename Op>
__device__ __forceinline__ T fold_waves(const T *red, T id, Op op) {
  const int w = threadIdx.x & 15;
  return row_fold(w < kWaves ? red[w] : id, op);
}
// The same for one value per wave (v: the wave's), written to red first:
// one barrier. red: LDS of its own per call site.
template <typename T, typename Op>
__device__ __forceinline__ T block_fold(T v, T *red, T id, Op op) {
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fold_waves(red, id, op);
}

template <bool kMass, int kPerThread>
__global__ __launch_bounds__(kThreads) void k_post_die(
    PoolParams p, DieTable t, double param, const float *__restrict__ imp,
    const int32_t *__restrict__ ids, float *__restrict__ token_scores,
    float *__restrict__ chunk_scores, uint8_t *__restrict__ keep, int32_t *__restrict__ n_kept,
    int32_t *__restrict__ kept_ids, int32_t *__restrict__ kept_pos,
    int64_t *__restrict__ kept_offsets, DieWs ws) {
  __shared__ __align__(16) float buf[kDieMaxTB + 2 * kHalo];
  __shared__ float xs[kDieMaxTB];
  __shared__ float gmin[kPostMaxGroups];                      // the prompt's pool-group mins
  __shared__ uint32_t bmn[kRangeGroups], bmx[kRangeGroups];   // the range's groups
  __shared__ float xpart[kDieMaxTB / 8 + kDieMaxChunks];     // chunk sums by runs of 8
  __shared__ uint32_t hcnt[kBins];
  __shared__ unsigned long long hmass[kMass ? kBins : 1];
  __shared__ SelState sst;
  __shared__ float red_lo[kWaves], red_hi[kWaves], red_mx[kWaves];
  __shared__ long long red_tot[kWaves], red_base[kWaves];
  __shared__ uint32_t red_omn[kWaves], red_omx[kWaves];
  __shared__ int red_before[kWaves], red_scan[kWaves];
  __shared__ uint8_t kraw[kScanPer * kThreads];    // the write part's chunks: kept, not final
  __shared__ uint8_t kflag[kScanPer * kThreads];   // kept (the final chunk included)
  __shared__ int kpre[kScanPer * kThreads];        // kept non-final chunks ahead of each
  __shared__ long long fx_last;           // the prompt's final chunk in fixed point
  __shared__ int keep0;                   // chunk 0 kept
  const int cta = blockIdx.x, d = cta % kXcds, rg = cta / kXcds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bool dead = false;
  if (cta == 0 && tid == 0) ws.hdr[1] = ws.tag;
  int b = 0;
  {
    int lo = 0, hi = t.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (t.rng_off[mid] <= rg) lo = mid; else hi = mid - 1;
    }
    b = lo;
  }
  const int64_t tok0 = t.tok_off[b];
  const int N = t.tok_off[b + 1] - t.tok_off[b];
  const int t0 = (rg - t.rng_off[b]) * t.TB, t1 = min(N, t0 + t.TB);
  const int c0 = t.chunk_off[b], nc = t.chunk_off[b + 1] - c0, last = nc - 1;
  const int ca = t0 / p.C, nck = (t1 - t0 + p.C - 1) / p.C;   // the range's chunks
  const int GT = t.GT;                                         // tokens per pool group
  const int q0 = t.grp_off[b], nq = t.grp_off[b + 1] - q0;     // the prompt's groups
  const int qa = t0 / GT, nqb = (t1 - t0 + GT - 1) / GT;       // the range's groups
  const bool first_range = rg == t.rng_off[b];

  // 1. Pooled values of the range (as k_pool_finish), each pool group's min
  //    and max, and each chunk's boosted sum relative to its group's min.
  {
    const int r = (p.W - 1) / 2;
    // The W = 13 form when pool groups hold whole 256-token waves: four
    // consecutive tokens per lane, the importance zero-padded outside the
    // prompt (LDS index of token x: x - t0 + kPad), so that the four
    // windows are one aligned 64-byte read and 13 adds each (a term
    // outside the prompt adds 0, as in window_mean).
    constexpr int kPad = 10;   // >= 6, and 16-byte alignment of each quad's window
    const bool quad = r == kDefaultPoolRadius && GT % 256 == 0;
    const int lo = quad ? t0 - kPad : max(0, t0 - r);
    const int hi = quad ? t1 + kPad : min(N, t1 + r);
    {
      // Every load in flight before any is stored.
      constexpr int kLd = (kDieMaxTB + 2 * kHalo + kThreads - 1) / kThreads;
      float v[kLd];
#pragma unroll
      for (int u = 0; u < kLd; ++u) {
        const int x = lo + tid + u * kThreads;
        v[u] = (x < hi && x >= 0 && x < N) ? imp[tok0 + x] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kLd; ++u) {
        const int i = tid + u * kThreads;
        if (i < hi - lo) buf[i] = v[u];
      }
    }
    if (tid < nqb) {
      bmn[tid] = ord_of(INFINITY);
      bmx[tid] = ord_of(-INFINITY);
    }
    if (tid < kBins) {   // the radix bins (first used in step 3)
      hcnt[tid] = 0u;
      if (kMass) hmass[tid] = 0ull;
    }
    __syncthreads();
    if (quad) {
      for (int qt = t0 + 4 * tid; qt - 4 * lane < t1; qt += 4 * kThreads) {   // (wave-uniform)
        float w[16];
        if (qt < t1) {
          const float4 *src = reinterpret_cast<const float4 *>(&buf[qt - 6 - lo]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4 f = src[i];
            w[4 * i] = f.x;
            w[4 * i + 1] = f.y;
            w[4 * i + 2] = f.z;
            w[4 * i + 3] = f.w;
          }
        }
        float mn4 = INFINITY, mx4 = -INFINITY;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int q = qt + u;
          if (q < t1) {
            float sum = 0.f;
#pragma unroll
            for (int k = 0; k < 13; ++k) sum += w[u + k];
            const int a = max(0, q - kDefaultPoolRadius), e = min(N - 1, q + kDefaultPoolRadius);
            const float x = sum / (float)(e - a + 1);
            xs[q - t0] = x;
            mn4 = fminf(mn4, x);
            mx4 = fmaxf(mx4, x);
          }
        }
        const float wmn = wave_min(mn4), wmx = wave_max(mx4);
        if (lane == 0) {   // the wave's 256 tokens lie in one pool group
          const int g = div_by(t.by_gt, qt - t0);
          atomicMin(&bmn[g], ord_of(wmn));
          atomicMax(&bmx[g], ord_of(wmx));
        }
      }
    } else {
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
              const int g = div_by(t.by_gt, wt - t0);
              atomicMin(&bmn[g], ord_of(wmn));
              atomicMax(&bmx[g], ord_of(wmx));
            }
          }
        } else if (tt < t1) {
          const int g = div_by(t.by_gt, tt - t0);
          atomicMin(&bmn[g], ord_of(x));
          atomicMax(&bmx[g], ord_of(x));
        }
      }
    }
    __syncthreads();
  }
  if (tid < nqb) {
    post(ws, d, 2 * (q0 + qa + tid), __float_as_uint(float_of(bmn[tid])));
    post(ws, d, 2 * (q0 + qa + tid) + 1, __float_as_uint(float_of(bmx[tid])));
  }
  {
    // Each chunk's runs of 8 tokens on lanes of their own, then the partials
    // in order (as chunk_rel adds them).
    const int runs = (p.C + 7) / 8;   // per chunk
    for (int w0 = 0; w0 < nck * runs; w0 += kThreads) {
      const int k = w0 + tid, c = div_by(t.by_runs, k), u = k - c * runs;
      if (k < nck * runs) {
        const int a = t0 + c * p.C, e = min(t1, a + p.C);
        xpart[k] = a + 8 * u < e
                       ? chunk_part(p, N, xs, t0, a + 8 * u, e, float_of(bmn[div_by(t.by_cpg, c)]))
                       : 0.f;
      }
    }
    __syncthreads();
    for (int c = tid; c < nck; c += kThreads) {
      const int a = t0 + c * p.C, e = min(t1, a + p.C);
      float rel = 0.f;
      for (int u = 0; a + 8 * u < e; ++u) rel = __fadd_rn(rel, xpart[c * runs + u]);
      post(ws, d, ws.cs0 + c0 + ca + c, __float_as_uint(rel));
    }
  }

  const int ept = (nc + kThreads - 1) / kThreads;   // sc[] slots in use (uniform)

  // 2. Every group's min and max and every chunk's sum of the prompt: the
  //    prompt's min and max and every chunk score (chunk tid + kThreads * e
  //    in sc[e]).
  float sc[kPerThread];
  float mn = 0.f, range = 1.f;
  bool flat = false;
  {
    constexpr int kQ = kPostMaxGroups / kThreads;   // groups per thread
    uint32_t got[2 * kQ + kPerThread];
    take(
        [&](int m) -> int64_t {
          if (m < 2 * kQ) {
            const int k = tid + kThreads * (m >> 1);
            return 2 * (q0 + (k < nq ? k : 0)) + (m & 1);
          }
          const int j = tid + kThreads * (m - 2 * kQ);
          return ws.cs0 + c0 + (j < nc ? j : 0);
        },
        [&](int m) {
          return m < 2 * kQ ? tid + kThreads * (m >> 1) < nq : tid + kThreads * (m - 2 * kQ) < nc;
        },
        got, ws, d, dead);
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
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) {
      red_lo[wave] = lo;
      red_hi[wave] = hi;
    }
    __syncthreads();   // (also publishes gmin)
    lo = fold_waves(red_lo, INFINITY, [](float a, float c) { return fminf(a, c); });
    hi = fold_waves(red_hi, -INFINITY, [](float a, float c) { return fmaxf(a, c); });
    if (p.normalize) {
      mn = lo;
      range = hi - lo;
      flat = range <= 1e-6f * hi;   // no signal: every score becomes 1
    }
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int j = tid + kThreads * e;
      sc[e] = 0.f;
      if (e < ept && j < nc) {
        const int a = j * p.C, en = min(N, a + p.C);
        sc[e] = chunk_score(__uint_as_float(got[2 * kQ + e]), boost_sum(p, N, a, en), gmin[div_by(t.by_cpg, j)],
                            en - a, p.normalize, flat, mn, range);
      }
    }
  }

  // 3. The selection: the prompt's fixed point, the threshold, then the
  //    number R of non-final chunks kept and the cutoff key (kept: key >>
  //    thr_sh <= thr_P) from a radix select. A chunk i ahead of the final
  //    one is kept when the chunks ahead of it in the order hold less than
  //    the threshold (mass: their fixed-point sum; top-p: their count), so
  //    the kept ones are the R smallest keys, and the last of them lies in
  //    the last bin (of candidates, by key) whose smallest key still passes.
  float mx = 0.f;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) mx = fmaxf(mx, sc[e]);
  mx = block_fold(wave_max(mx), red_mx, 0.f, [](float a, float c) { return fmaxf(a, c); });
  const int shift = fixed_shift(mx);
  // Each chunk's fixed-point score and key, kept in registers up to 8 per
  // thread (beyond, recomputed where needed). sc[e] is 0 past the prompt's
  // chunks.
  constexpr bool kKeep = kPerThread <= 8;
  long long fxa[kKeep ? kPerThread : 1];
  unsigned long long cka[kKeep ? kPerThread : 1];
  auto fx = [&](int e) -> long long {
    if constexpr (kKeep) return fxa[e]; else return to_fixed(sc[e], shift);
  };
  auto key = [&](int e) -> unsigned long long {
    if constexpr (kKeep) return cka[e]; else return chunk_key(fx(e), tid + kThreads * e);
  };
  long long tot = 0;                              // fixed-point sum of the thread's chunks
  uint32_t omn = ~0u, omx = 0u;                   // its non-final chunks' score keys
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    if (e < ept) {
      const int j = tid + kThreads * e;
      const long long f = to_fixed(sc[e], shift);
      const unsigned long long ck = chunk_key(f, j);
      if constexpr (kKeep) {
        fxa[e] = f;
        cka[e] = ck;
      }
      tot += f;
      if (j == last) fx_last = f;
      if (j < last) {
        const uint32_t ok = (uint32_t)(ck >> (kKeyBits - 32));
        omn = min(omn, ok);
        omx = max(omx, ok);
      }
    }
  }
  // Adds the candidates of a radix pass (keys k with k >> s.top == s.P) to
  // the bins of their digit, bits [s.sh, s.top): counts and fixed-point sums.
  auto add_bins = [&](const SelState &s) {
    const uint32_t dmask = (1u << (s.top - s.sh)) - 1u;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (e < ept) {   // (uniform)
        const int j = tid + kThreads * e;
        const long long f = fx(e);
        const unsigned long long ck = key(e);
        const bool act = j < last && (ck >> s.top) == s.P;
        const uint32_t bin = (uint32_t)(ck >> s.sh) & dmask;
        const unsigned long long am = __ballot(act);
        if (am) {
          // A wave whose candidates share one bin adds them as one.
          const int fl = __builtin_ctzll(am);
          const uint32_t fb = (uint32_t)__builtin_amdgcn_readlane((int)bin, fl);
          if (__ballot(act && bin != fb) == 0) {
            const long long ms = kMass ? wave_sum_i64(act ? f : 0ll) : 0ll;
            if (lane == 0) {
              atomicAdd(&hcnt[fb], (uint32_t)__popcll(am));
              if (kMass) atomicAdd(&hmass[fb], (unsigned long long)ms);
            }
          } else if (act) {
            atomicAdd(&hcnt[bin], 1u);
            if (kMass) atomicAdd(&hmass[bin], (unsigned long long)f);
          }
        }
      }
    }
  };
  // The first pass's bins at once, on the top digit of the keys: the first
  // digit whenever two non-final chunks' scores differ in their top bit,
  // which is the usual case (checked below). The adds overlap the
  // reductions and need no barrier of their own.
  SelState s0 = {0ull, 0ll, 0, kKeyBits - 8, kKeyBits, 0};
  if (last > 1) add_bins(s0);
  tot = wave_sum_i64(tot);
  const auto umin = [](uint32_t a, uint32_t c) { return a < c ? a : c; };
  const auto umax = [](uint32_t a, uint32_t c) { return a > c ? a : c; };
  omn = wave_reduce_u32(omn, umin);
  omx = wave_reduce_u32(omx, umax);
  if (lane == 0) {
    red_tot[wave] = tot;
    red_omn[wave] = omn;
    red_omx[wave] = omx;
  }
  __syncthreads();   // (also publishes fx_last)
  tot = fold_waves(red_tot, 0ll, [](long long a, long long c) { return a + c; });
  omn = fold_waves(red_omn, ~0u, umin);
  omx = fold_waves(red_omx, 0u, umax);
  // Every non-final chunk's key lies in [kmn, kmx], and the smallest and
  // largest of them agree with these bounds on their score part, so the
  // highest bit in which the bounds differ is that of the keys whenever
  // two scores differ (else it lies in the index part, and the select
  // takes one digit more at most).
  const unsigned long long kmn = (unsigned long long)omn << (kKeyBits - 32);
  const unsigned long long kmx = ((unsigned long long)omx << (kKeyBits - 32)) |
                                 ((1ull << (kKeyBits - 32)) - 1ull);
  const long long need = kMass ? (long long)ceil(param * (double)tot) - fx_last
                               : (long long)(t.kc[b] - 1);   // chunks ahead of a kept one
  int R = 0, thr_sh = 0;
  unsigned long long thr_P = 0;
  if (last > 0 && need > 0) {
    if (last == 1) {
      R = 1;   // one non-final chunk: nothing is ahead of it
      thr_sh = kKeyBits;   // every key >> kKeyBits is 0 = thr_P
    } else {
      // The first digit: the highest 8 bits in which the keys differ. When
      // that is the top digit its bins are filled already; else they start
      // again from zero.
      const int hb = 63 - __builtin_clzll(kmn ^ kmx);
      SelState s = {kmn >> (hb + 1), 0ll, 0, max(0, hb - 7), hb + 1, 0};
      bool pre = hb == kKeyBits - 1;
      if (!pre) {
        if (tid < kBins) {
          hcnt[tid] = 0u;
          if (kMass) hmass[tid] = 0ull;
        }
        __syncthreads();
      }
      for (;;) {
        if (!pre) {
          add_bins(s);
          __syncthreads();
        }
        pre = false;
        if (wave == 0) {
          // Lane l holds bins 4 l .. 4 l + 3 (ascending keys); exclusive
          // prefixes of their counts and sums over the bins.
          uint32_t cc[4];
          long long mm[4];
          uint32_t lc = 0;
          long long lm = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            cc[i] = hcnt[4 * lane + i];
            mm[i] = kMass ? (long long)hmass[4 * lane + i] : 0ll;
            lc += cc[i];
            lm += mm[i];
          }
          uint32_t ec = wave_scan_u32(lc) - lc;
          long long em = kMass ? wave_scan_i64(lm) - lm : 0ll;
          int best = -1;
          uint32_t bec = 0, bcnt = 0;
          long long bem = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = cc[i] > 0 && (kMass ? s.bm + em < need : (long long)(s.bc + (int)ec) < need);
            if (ok) {
              best = 4 * lane + i;
              bec = ec;
              bem = em;
              bcnt = cc[i];
            }
            ec += cc[i];
            em += mm[i];
          }
          const int bs = (int)wave_reduce_u32((uint32_t)(best + 1),
                                              [](uint32_t a, uint32_t c) { return a > c ? a : c; }) - 1;
          if (best == bs && bs >= 0) {
            SelState n = s;
            n.bc = s.bc + (int)bec;
            n.bm = s.bm + bem;
            n.P = (s.P << (s.top - s.sh)) | (unsigned long long)bs;
            n.top = s.sh;
            n.sh = max(0, s.sh - 8);
            n.done = bcnt == 1 || s.sh == 0;
            if (n.done) n.sh = s.sh;   // the cutoff's level
            sst = n;
          } else if (bs < 0 && lane == 0) {
            // (Cannot happen: the smallest candidate always passes. Stop with
            // no chunk kept rather than loop.)
            SelState n = s;
            n.done = 1;
            n.bc = -1;
            sst = n;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hcnt[4 * lane + i] = 0u;
            if (kMass) hmass[4 * lane + i] = 0ull;
          }
        }
        __syncthreads();
        s = sst;
        if (s.done) break;
      }
      R = s.bc + 1;
      thr_sh = s.sh;
      thr_P = s.P;
    }
  }
  auto kept = [&](int e) -> bool {
    const int j = tid + kThreads * e;
    if (j == last) return true;
    return R > 0 && j < last && (key(e) >> thr_sh) <= thr_P;
  };

  // 4. This die's eighth of the range: tokens [u0, u1), chunks [cu0, cu1).
  const int sub = (t.TB + kXcds - 1) / kXcds;
  const int u0 = min(t1, t0 + d * sub), u1 = min(t1, u0 + sub);
  const int cu0 = u0 / p.C, cu1 = u1 > u0 ? (u1 - 1) / p.C + 1 : cu0;
  const int ncu = cu1 - cu0;
  // Kept non-final chunks ahead of cu0; the flags of [cu0, cu1) to LDS,
  // then their exclusive prefix: from one ballot in every wave when the
  // part has at most 64 chunks (16 at 4096-token ranges and C = 32), else
  // by a block scan into kpre.
  int before = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    if (e < ept) {
      const int j = tid + kThreads * e;
      if (j < nc) {
        const bool k = kept(e);
        if (j < cu0 && j < last && k) ++before;
        if (j >= cu0 && j < cu1) {
          kraw[j - cu0] = (k && j < last) ? 1 : 0;
          kflag[j - cu0] = k ? 1 : 0;
        }
        if (j == 0) keep0 = k ? 1 : 0;
      }
    }
  }
  before = (int)wave_reduce_u32((uint32_t)before, [](uint32_t a, uint32_t c) { return a + c; });
  if (lane == 0) red_before[wave] = before;
  __syncthreads();
  const bool small = ncu <= 64;   // (uniform)
  int before_all = 0;
  unsigned long long kmask = 0;   // the part's kept non-final chunks, one bit each
  if (small) {
    const int w16 = lane & 15;
    before_all = row_fold(w16 < kWaves ? red_before[w16] : 0, [](int a, int c) { return a + c; });
    kmask = __ballot(lane < ncu && kraw[lane] != 0);
  } else {
    // Thread tid takes chunks kScanPer tid .. + kScanPer - 1 of the part.
    int v[kScanPer], sum = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      const int c = kScanPer * tid + i;
      v[i] = c < ncu ? kraw[c] : 0;
      sum += v[i];
    }
    const int incl = (int)wave_scan_u32((uint32_t)sum);
    if (lane == 63) red_scan[wave] = incl;
    __syncthreads();
    const int w16 = lane & 15;
    int pre = row_fold(w16 < kWaves ? red_before[w16] + (w16 < wave ? red_scan[w16] : 0) : 0,
                       [](int a, int c) { return a + c; }) +
              incl - sum;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      const int c = kScanPer * tid + i;
      if (c < ncu) kpre[c] = pre;
      pre += v[i];
    }
  }
  const bool bos = keep0 == 0;
  // Kept tokens of the prompt: BOS when chunk 0 is dropped, R whole chunks
  // and the final chunk.
  const long long total_b = (bos ? 1 : 0) + (long long)R * p.C + (N - last * p.C);
  long long base = 0;   // the prompt's first packed position
  if (t.B > 1) {
    if (first_range && tid == 0) post(ws, d, ws.cnt0 + b, (uint32_t)total_b);
    uint32_t got[1];
    take([&](int) -> int64_t { return ws.cnt0 + (tid < b ? tid : 0); },
         [&](int) { return tid < b; }, got, ws, d, dead);
    base = block_fold(wave_sum_i64(tid < b ? (long long)got[0] : 0ll), red_base, 0ll,
                      [](long long a, long long c) { return a + c; });
  } else if (!small) {
    __syncthreads();   // kpre
  }
  // Kept non-final chunks ahead of chunk cu0 + i.
  auto ahead = [&](int i) -> long long {
    return small ? (long long)(before_all + __popcll(kmask & ((1ull << i) - 1ull))) : (long long)kpre[i];
  };
  // Chunk scores, keep flags and token scores of the write part.
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    if (e < ept) {
      const int j = tid + kThreads * e;
      if (j < nc && j * p.C >= u0 && j * p.C < u1) {
        chunk_scores[c0 + j] = sc[e];
        keep[c0 + j] = kept(e) ? 1 : 0;
      }
    }
  }
  if (token_scores) {
    for (int tt = u0 + tid; tt < u1; tt += kThreads) {
      float x = xs[tt - t0];
      if (p.normalize) x = flat ? 1.f : (x - mn) / range;
      token_scores[tok0 + tt] = boosted(p, N, tt, x);
    }
  }
  if (first_range && d == 0 && tid == 0) n_kept[b] = R + 1;
  // A wait that ran out anywhere in the block leaves the positions unknown:
  // then nothing is written at a position they would give.
  if (__syncthreads_or(dead ? 1 : 0)) return;
  const int64_t total = t.tok_off[t.B];
  if (first_range && d == 0 && tid == 0) {
    kept_offsets[b] = base;
    if (b == t.B - 1) kept_offsets[t.B] = base + total_b;
  }
  if (bos && u0 == 0 && u1 > 0 && tid == 0 && base < total) {
    kept_ids[base] = ids[tok0];
    kept_pos[base] = 0;
  }
  const long long first = base + (bos ? 1 : 0);
  for (int tt = u0 + tid; tt < u1; tt += kThreads) {
    const int c = ca + div_by(t.by_c, tt - t0);
    if (!kflag[c - cu0]) continue;
    const long long out = first + ahead(c - cu0) * p.C + (tt - c * p.C);
    if (out >= total) continue;
    kept_ids[out] = ids[tok0 + tt];
    kept_pos[out] = tt;
  }
}

}  // namespace

int post_die_ranges() {
  constexpr int kMaxDevices = 64;
  static int ranges[kMaxDevices];
  static bool done[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!done[dev]) {
    done[dev] = true;
    auto fits = [](auto kern) {
      int n = 0;
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, kThreads, 0) == hipSuccess && n >= 1;
    };
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus >= kXcds && cus % kXcds == 0 &&
        fits(k_post_die<true, kMinEPT>) && fits(k_post_die<false, kMinEPT>) &&
        fits(k_post_die<true, 2 * kMinEPT>) && fits(k_post_die<false, 2 * kMinEPT>) &&
        fits(k_post_die<true, kMaxEPT>) && fits(k_post_die<false, kMaxEPT>))
      ranges[dev] = cus / kXcds;
  }
  return ranges[dev];
}

size_t post_die_slot_bytes(int B, int total_chunks, int total_groups) {
  const size_t per = align_up(((size_t)2 * total_groups + total_chunks + B) * sizeof(uint64_t));
  return 2 * kXcds * per;
}

hipError_t launch_post_die(int mode, double param, const PoolParams &p, const DieTable &t,
                           const float *imp, const int32_t *ids, float *token_scores,
                           float *chunk_scores, uint8_t *keep, int32_t *n_kept, int32_t *kept_ids,
                           int32_t *kept_pos, int64_t *kept_offsets, void *ws, hipStream_t st) {
  DieWs w;
  char *base = reinterpret_cast<char *>(ws);
  w.hdr = reinterpret_cast<uint32_t *>(base);
  w.slots = reinterpret_cast<uint64_t *>(base + kStatusBytes);
  const int G = t.grp_off[t.B], NC = t.chunk_off[t.B];
  w.per = (int64_t)(align_up(((size_t)2 * G + NC + t.B) * sizeof(uint64_t)) / sizeof(uint64_t));
  w.cs0 = 2 * (int64_t)G;
  w.cnt0 = w.cs0 + NC;
  w.tag = reserve_tags(1);
  w.wait_ticks = score_wait_ticks();
  const int grid = kXcds * t.NR;
  int most = 0;
  for (int b = 0; b < t.B; ++b) most = std::max(most, t.chunk_off[b + 1] - t.chunk_off[b]);
  const bool mass = mode == SP_SELECT_MASS;
  auto kern = most <= kMinEPT * kThreads
                  ? (mass ? k_post_die<true, kMinEPT> : k_post_die<false, kMinEPT>)
              : most <= 2 * kMinEPT * kThreads
                  ? (mass ? k_post_die<true, 2 * kMinEPT> : k_post_die<false, 2 * kMinEPT>)
                  : (mass ? k_post_die<true, kMaxEPT> : k_post_die<false, kMaxEPT>);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, st, p, t, param, imp, ids, token_scores,
                     chunk_scores, keep, n_kept, kept_ids, kept_pos, kept_offsets, w);
  return hipGetLastError();
}

}  // namespace sp
