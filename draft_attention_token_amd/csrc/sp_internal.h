// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specprefill.h"

namespace sp {

constexpr int kTile = 32;          // keys per MFMA tile (the 32-wide N of 32x32 MFMA)
constexpr int kRows = 32;          // query rows per MFMA tile: (lookahead step, head in group)
constexpr size_t kAlign = 256;
// The scoring workspace starts with a 256-byte header of two uint32 tags:
// [1] is the tag of the latest call, [0] the tag of a call in which a
// cross-block wait timed out. Every call gets fresh tags (reserve_tags).
constexpr size_t kStatusBytes = 256;
constexpr float kLog2e = 1.4426950408889634f;
// Pool-before-max: probabilities of kPoolHalo keys each side of a 32-key
// output tile are on chip, so a row pool reaches at most that far.
constexpr int kPoolHalo = 16;
constexpr int kPoolSpan = 64;                     // kTile + 2 * kPoolHalo
constexpr int kMaxRowPool = 2 * kPoolHalo + 1;
constexpr int kDefaultPoolRadius = 6;   // W = 13 ("Speculative prefill", Approach step 3)

// Per-prompt prefix table passed to kernels by value (about 1 KB). unit_off
// holds a host-computed prefix of per-prompt unit counts (tiles, chunks or
// token blocks, depending on the kernel); tok_off the prompt token offsets
// (the library rejects batches of 2^31 tokens or more).
struct SegTable {
  int32_t B;
  int32_t L;                          // lookahead keys per prompt (0 where unused)
  int32_t unit_off[SP_MAX_PROMPTS + 1];
  int32_t tok_off[SP_MAX_PROMPTS + 1];
};

// Prompt that owns global unit u (unit_off is non-decreasing, u < unit_off[B]).
__device__ __forceinline__ int seg_of(const SegTable &t, int32_t u) {
  int lo = 0, hi = t.B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (t.unit_off[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Reduction with op over the 64 lanes of a wave, the result in every lane:
// DPP within each row of 16 lanes (lane xor 1 and xor 2 by quad permutes,
// then rotations by 4 and 8 gather the row's four quads), then the four row
// values read as scalars. Few-cycle steps, where a lane shuffle is an LDS
// crossbar round trip. op must be associative and commutative.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, false));   // xor 1
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xf, 0xf, false));   // xor 2
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xf, 0xf, false));  // ror 4
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xf, 0xf, false));  // ror 8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ float wave_min(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
// Block-wide forms (kWaves waves; red: kWaves entries of LDS), the result
// in every thread; they synchronise the block.
template <int kWaves>
__device__ __forceinline__ float block_max(float v, float *red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) v = fmaxf(v, red[w]);
  __syncthreads();
  return v;
}
template <int kWaves>
__device__ __forceinline__ float2 block_minmax(float lo, float hi, float2 *red) {
  lo = wave_min(lo);
  hi = wave_max(hi);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_float2(lo, hi);
  __syncthreads();
  float2 v = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    v.x = fminf(v.x, red[w].x);
    v.y = fmaxf(v.y, red[w].y);
  }
  __syncthreads();
  return v;
}
// Sum over the wave of a 64-bit integer (exact), in every lane.
__device__ __forceinline__ long long wave_sum_i64(long long v) {
  unsigned long long x = (unsigned long long)v;
#define SP_DPP_ADD64(ctrl)                                                                        \
  {                                                                                               \
    const uint32_t l2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, ctrl, 0xf, 0xf, false); \
    const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), ctrl, 0xf, 0xf, false); \
    x += ((unsigned long long)h2 << 32) | l2;                                                     \
  }
  SP_DPP_ADD64(0xB1) SP_DPP_ADD64(0x4E) SP_DPP_ADD64(0x124) SP_DPP_ADD64(0x128)
#undef SP_DPP_ADD64
  unsigned long long t = 0;
#pragma unroll
  for (int r = 0; r < 64; r += 16)
    t += ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), r) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, r);
  return (long long)t;
}
template <int kWaves>
__device__ __forceinline__ long long block_sum(long long v, long long *red) {
  v = wave_sum_i64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) v += red[w];
  __syncthreads();
  return v;
}

// Output offsets of a batch's prompts from their kept counts, on one wave
// (lane l takes prompts 2 l and 2 l + 1; B <= SP_MAX_PROMPTS = 128): returns
// the offset of prompt b to every lane, and when `offsets` is not null
// writes offsets[0 .. B] (offsets[B] = the total). Counts sum below 2^31.
__device__ __forceinline__ int64_t wave_prompt_offsets(const int32_t *counts, int B, int b,
                                                       int64_t *offsets) {
  const int lane = threadIdx.x & 63, i0 = 2 * lane, i1 = i0 + 1;
  const int c0 = i0 < B ? counts[i0] : 0, c1 = i1 < B ? counts[i1] : 0;
  const int pair = c0 + c1;
  int incl = pair;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  const int e0 = incl - pair, e1 = e0 + c0;   // offsets of prompts i0 and i1
  if (offsets) {
    if (i0 <= B) offsets[i0] = e0;
    if (i1 <= B) offsets[i1] = e1;
    if (lane == 63) offsets[B] = incl;   // the total (B = 128 has no lane of its own)
  }
  const int mine = i0 == b ? e0 : (i1 == b ? e1 : 0);
  int v = (i0 == b || i1 == b) ? mine : 0;
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
static_assert(SP_MAX_PROMPTS <= 128, "two prompts per lane of one wave");

// The selection's fixed point and order: floor(v * 2^shift) from the
// float's bits (exact, no floating-point rounding), the shift set by the
// prompt's largest score so that it lands in [2^47, 2^48); chunks are
// ranked on the top 32 bits of that value, an ascending key being a
// descending score.
__device__ __forceinline__ int fixed_shift(float mx) {
  int e = 0;
  if (mx > 0.f) frexpf(mx, &e);   // mx < 2^e
  return 48 - e;
}
// For finite v >= 0 with v * 2^shift < 2^63.
__device__ __forceinline__ long long to_fixed(float v, int shift) {
  const uint32_t u = __float_as_uint(v);
  const int e = (int)((u >> 23) & 0xffu);
  const unsigned long long m = (u & 0x7fffffu) | (e ? 0x800000u : 0u);
  const int sh = (e ? e : 1) - 150 + shift;   // v = m * 2^((e ? e : 1) - 150)
  if (sh >= 0) return (long long)(m << sh);
  return sh <= -64 ? 0ll : (long long)(m >> (-sh));
}
__device__ __forceinline__ uint32_t order_key(long long fx) {
  return 0xffffffffu - (uint32_t)((unsigned long long)fx >> 16);
}
// Ordered-integer image of a float (monotone): LDS atomics take min and max.
__device__ __forceinline__ uint32_t ord_of(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_of(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

struct AttnShape {
  int n_layers, Hq, Hkv, d;
  int L;                            // query steps per (layer, head): La + pre
  int G;
  int La;                           // lookahead keys per prompt (K rows past the prompt)
  int pre;                          // 1: step 0 is the prompt's last row (position N - 1)
  int row_pool;                     // 1, or odd W > 1: pool each probability row first
  float scale_log2;                 // scale * log2(e): logits kept in base-2 units
  int dtype;
};

// n consecutive nonzero tags, unique within the process (until 2^32 calls).
uint32_t reserve_tags(int n);
// Budget of a cross-block wait in wall-clock ticks (100 MHz): 2 s, or
// SP_SCORE_WAIT_US microseconds when that is set.
uint64_t score_wait_ticks();

// Launchers (return hipError_t of the launch).
// Scoring workspace: header, then the single-pass kernel's slots (for shapes
// it supports), then the two-pass kernel's region; one layout for every algo.
hipError_t launch_score_two_pass(const AttnShape &s, const SegTable &tiles, int total_tiles,
                                 const void *q, const void *k, float *imp, uint32_t *hdr,
                                 void *region, hipStream_t st);
size_t score_two_pass_region_bytes(const AttnShape &s, int B, int total_tiles);

bool score_stream_supported(const AttnShape &s);
size_t score_stream_slot_bytes(const AttnShape &s);
// Per-problem multipliers of the logit scale for fp8 K (problem x = layer *
// Hkv + group); unused for other K types.
constexpr int kMaxScaledProblems = 128;
struct KScales {
  float v[kMaxScaledProblems];
};
// Sets *supported = false (and launches nothing) when the device or the
// batch does not fit the kernel.
hipError_t launch_score_stream(const AttnShape &s, const SegTable &tiles, const void *q,
                               const void *k, const KScales &ks, float *imp, void *ws,
                               hipStream_t st, bool *supported);
// Whether the single pass takes the batch on the current device, and if so
// its number of launches and each prompt's launch (prompt_launch may be null).
bool score_stream_plan(const AttnShape &s, const SegTable &tiles, int *n_launches,
                       int32_t *prompt_launch);

// Mean of buf over the window of token t clipped to the prompt, summed in
// token order. R >= 0: the radius at compile time (the loads issue together);
// R < 0: radius r at run time.
template <int R>
__device__ __forceinline__ float window_mean(const float *buf, int lo, int N, int t, int r) {
  const int a = max(0, t - r), e = min(N - 1, t + r);
  float sum = 0.f;
  if constexpr (R >= 0) {
#pragma unroll
    for (int k = -R; k <= R; ++k) {
      const int i = t + k;
      const float v = buf[min(max(i, a), e) - lo];   // always inside the staged span
      sum += (i >= a && i <= e) ? v : 0.f;
    }
  } else {
    for (int i = a; i <= e; ++i) sum += buf[i - lo];
  }
  return sum / (float)(e - a + 1);
}

struct PoolParams {
  int W, C, normalize, first_n, last_n;
  float first_mult, last_mult;
};

// v times the boosts of token t of a prompt of N tokens (first, then last;
// a factor of 1 where a boost does not apply leaves v as it is).
// The products and sums of these helpers are rounded one by one, so that
// every kernel that inlines them gets the same bits. The rounding helpers
// are plain operators, which the compiler may fuse into a multiply-add; a
// product passed through rounded() is opaque to it and is not fused.
__device__ __forceinline__ float rounded(float x) {
  asm("" : "+v"(x));
  return x;
}
__device__ __forceinline__ float boosted(const PoolParams &p, int N, int t, float v) {
  v = __fmul_rn(v, t < p.first_n ? p.first_mult : 1.f);
  return rounded(__fmul_rn(v, t >= N - p.last_n ? p.last_mult : 1.f));
}
// Sum of the boosts of tokens [a, e): the tokens with no boost, then those
// with the first boost only, the last boost only and both, each kind its
// count times its factor (e - a where none applies).
__device__ __forceinline__ float boost_sum(const PoolParams &p, int N, int a, int e) {
  if (a >= p.first_n && e <= N - p.last_n) return (float)(e - a);
  const int fe = min(e, p.first_n), l0 = max(a, N - p.last_n);
  const int nf = max(0, fe - a), nl = max(0, e - l0), nb = max(0, fe - l0);
  float s = (float)(e - a - nf - nl + nb);
  s = __fadd_rn(s, rounded(__fmul_rn((float)(nf - nb), p.first_mult)));
  s = __fadd_rn(s, rounded(__fmul_rn((float)(nl - nb), p.last_mult)));
  return __fadd_rn(s, rounded(__fmul_rn((float)nb, __fmul_rn(p.first_mult, p.last_mult))));
}
// Sum of b_t (x_t - g) over tokens [a, e), x_t at xs[t - base] (LDS), in a
// fixed order: partial sums of consecutive runs of 8 tokens, each in token
// order, then the partials in order (chunk_rel; chunk_part gives one run so
// that lanes can take them in parallel).
__device__ __forceinline__ float chunk_part(const PoolParams &p, int N, const float *xs, int base,
                                            int a, int e, float g) {
  float v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = xs[min(a + u, e - 1) - base];   // (clamped: unused past e)
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (a + u < e) s = __fadd_rn(s, boosted(p, N, a + u, v[u] - g));
  return s;
}
__device__ __forceinline__ float chunk_rel(const PoolParams &p, int N, const float *xs, int base,
                                           int a, int e, float g) {
  float rel = 0.f;
  for (int t = a; t < e; t += 8) rel = __fadd_rn(rel, chunk_part(p, N, xs, base, t, e, g));
  return rel;
}
// A chunk's score, the mean over its n tokens of their normalised, boosted
// scores b_t (x_t - mn) / range, from sums that do not need the prompt's
// min and max: rel = sum of b_t (x_t - g) in token order, with g the min of
// the chunk's pool group (so every term is >= 0), and bs = sum of b_t. The
// mean is (rel + (g - mn) bs) / (range n); without normalisation (mn = 0,
// range = 1) (rel + g bs) / n; a flat prompt (every score 1) bs / n.
__device__ __forceinline__ float chunk_score(float rel, float bs, float g, int n, bool normalize,
                                             bool flat, float mn, float range) {
  if (!normalize) return __fmaf_rn(g, bs, rel) / (float)n;
  if (flat) return bs / (float)n;
  return __fmaf_rn(g - mn, bs, rel) / (range * (float)n);
}
// Pooling works on blocks of whole chunks of one prompt,
// pool_block_tokens(C) = C * max(1, floor(256 / C)) tokens each; these
// blocks are also the pool groups whose min enters the chunk scores.
struct PoolTable {
  int32_t B;
  int32_t blk_off[SP_MAX_PROMPTS + 1];     // block prefix per prompt
  int32_t chunk_off[SP_MAX_PROMPTS + 1];   // chunk prefix per prompt
  int32_t tok_off[SP_MAX_PROMPTS + 1];     // token offsets
};
int pool_block_tokens(int C);
hipError_t launch_pool_chunk(const PoolParams &p, const PoolTable &blocks, const float *imp,
                             float *token_scores, float *chunk_scores, void *ws, hipStream_t st);
constexpr int kMaxPoolWindow = 129;
size_t pool_ws(int B, int total_blocks);

// Chunk selection tables (host-computed), passed by value.
struct SelectTable {
  int32_t B;
  int32_t chunk_off[SP_MAX_PROMPTS + 1];   // chunk prefix per prompt
  int32_t blk_off[SP_MAX_PROMPTS + 1];     // rank-kernel block prefix per prompt
  int32_t kc[SP_MAX_PROMPTS];              // top-p budget per prompt
};
int select_rank_blocks(int nc);
// (The selection needs no workspace.)
hipError_t launch_select(int mode, double param, const SelectTable &t, const float *chunk_scores,
                         uint8_t *keep, int32_t *n_kept, hipStream_t st);

// Pooling, selection and compaction in one launch (post.hip): blocks of TB
// tokens (whole pool groups of one prompt, at most kPostMaxTB tokens and
// kPostMaxChunks chunks), at most one per CU and kPostMaxBlocks in all, all
// resident at once; at most kPostMaxGroups pool groups per prompt.
constexpr int kPostMaxTB = 2048;
constexpr int kPostMaxChunks = 64;
constexpr int kPostMaxBlocks = 1024;
constexpr int kPostMaxGroups = 2048;
struct PostTable {
  int32_t B, G, TB;
  int32_t GT;                              // tokens per pool group: pool_block_tokens(C)
  int32_t blk_off[SP_MAX_PROMPTS + 1];     // block prefix per prompt
  int32_t chunk_off[SP_MAX_PROMPTS + 1];   // chunk prefix per prompt
  int32_t grp_off[SP_MAX_PROMPTS + 1];     // pool-group prefix per prompt
  int32_t tok_off[SP_MAX_PROMPTS + 1];     // token offsets
  int32_t kc[SP_MAX_PROMPTS];              // top-p budget per prompt
};
// Blocks the fused launch may use on the current device (0: it cannot run).
int post_max_blocks();
// Bytes of its slots (after the status header) for a batch's chunks and
// pool groups.
size_t post_slot_bytes(int total_chunks, int total_groups);
hipError_t launch_post(int mode, double param, const PoolParams &p, const PostTable &t,
                       const float *imp, const int32_t *ids, float *token_scores,
                       float *chunk_scores, uint8_t *keep, int32_t *n_kept, int32_t *kept_ids,
                       int32_t *kept_pos, int64_t *kept_offsets, void *ws, hipStream_t st);
// The same in a launch whose blocks exchange values only with blocks of their
// own chip die (post_die.hip): every die runs the whole batch, cut into NR
// ranges of TB tokens (whole pool groups of one prompt, at most kDieMaxTB
// tokens and kDieMaxChunks chunks); block c takes range c / 8 and writes the
// eighth c % 8 of it. At most kDieMaxPrompts prompts and one range per CU
// of a die.
constexpr int kXcds = 8;                 // chip dies (XCDs); a launch deals block c to die c % 8
constexpr int kDieMaxTB = 8192;
constexpr int kDieMaxChunks = 1024;
constexpr int kDieMaxPrompts = 32;
// Division by a divisor fixed for a launch, by one high multiply: for
// d >= 1 and n (d - 1) < 2^32, floor(n / d) = hi32(n m) with m =
// ceil(2^32 / d), since m d - 2^32 < d keeps n m / 2^32 - n / d below
// 1 / d; d = 1 (m = 2^32) takes n itself. m comes from the host.
struct FastDiv {
  uint32_t m, one;
};
inline FastDiv fast_div(uint32_t d) {
  FastDiv f;
  f.m = (uint32_t)(((1ull << 32) + d - 1) / d);
  f.one = d == 1 ? ~0u : 0u;
  return f;
}
__device__ __forceinline__ int div_by(const FastDiv &f, int n) {
  return (int)(__umulhi((uint32_t)n, f.m) + ((uint32_t)n & f.one));
}

struct DieTable {
  int32_t B, NR, TB;
  int32_t GT;                                // tokens per pool group: pool_block_tokens(C)
  FastDiv by_gt, by_c, by_cpg, by_runs;      // / GT, / C, / (GT / C), / ceil(C / 8)
  int32_t rng_off[kDieMaxPrompts + 1];       // range prefix per prompt
  int32_t chunk_off[kDieMaxPrompts + 1];     // chunk prefix per prompt
  int32_t grp_off[kDieMaxPrompts + 1];       // pool-group prefix per prompt
  int32_t tok_off[kDieMaxPrompts + 1];       // token offsets
  int32_t kc[kDieMaxPrompts];                // top-p budget per prompt
};
// Ranges per die the die-local launch may use on the current device (0: it
// cannot run).
int post_die_ranges();
// Bytes of its slots (after the status header).
size_t post_die_slot_bytes(int B, int total_chunks, int total_groups);
hipError_t launch_post_die(int mode, double param, const PoolParams &p, const DieTable &t,
                           const float *imp, const int32_t *ids, float *token_scores,
                           float *chunk_scores, uint8_t *keep, int32_t *n_kept, int32_t *kept_ids,
                           int32_t *kept_pos, int64_t *kept_offsets, void *ws, hipStream_t st);
// Marks the status header at ws as a call with no timed-out wait.
hipError_t launch_stamp(void *ws, hipStream_t st);

hipError_t launch_gather(const SegTable &chunks, const SegTable &blocks, int total_blocks, int C,
                         const uint8_t *keep, const int32_t *ids, int32_t *kept_ids,
                         int32_t *kept_pos, int64_t *kept_offsets, void *ws, hipStream_t st);
constexpr int kGatherBlockTokens = 1024;
size_t gather_ws(int B, int total_chunks);

// Standalone-tool semantics (tool.hip).
struct StitchTable {
  int32_t n_windows;
  int32_t start[SP_MAX_PROMPTS];     // window's first token in the prompt
  int32_t keep[SP_MAX_PROMPTS];      // tokens of the window whose scores count
  int32_t win_off[SP_MAX_PROMPTS];   // window's offset in the window batch
};
hipError_t launch_stitch(const StitchTable &t, int32_t n, const float *win_imp, float *out,
                         hipStream_t st);

struct LegacyTable {
  int32_t B, C, max_keep;
  int32_t tok_off[SP_MAX_PROMPTS + 1];
  int32_t chunk_off[SP_MAX_PROMPTS + 1];
  int32_t blk_off[SP_MAX_PROMPTS + 1];     // rank-kernel block prefix per prompt
  int32_t wblk_off[SP_MAX_PROMPTS + 1];    // write-kernel block prefix per prompt
  int32_t kc[SP_MAX_PROMPTS];              // chunks ranked in (all of them: keep everything)
  int32_t eff_min[SP_MAX_PROMPTS];         // kept-token floor (0: none)
};
struct LegacyWs {
  uint8_t *in;            // [chunks] chunk kept by rank
  int32_t *kept_before;   // [chunks] kept tokens before the chunk (fill included)
  int32_t *rest_before;   // [chunks] tokens outside the base set before the chunk
  int32_t *counts;        // [B] kept tokens after the cap
  int32_t *stats;         // [B][2] kept tokens before the cap, fill
  size_t bytes;
};
LegacyWs legacy_ws(int B, int total_chunks, void *base);
int legacy_rank_blocks(int nc);
int legacy_write_blocks(int n);
hipError_t launch_legacy(const LegacyTable &t, const float *chunk_scores, const int32_t *ids,
                         void *ws, int32_t *kept_ids, int32_t *kept_pos, int64_t *kept_offsets,
                         hipStream_t st);

}  // namespace sp
