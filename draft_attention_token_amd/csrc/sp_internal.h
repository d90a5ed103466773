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

struct PoolParams {
  int W, C, normalize, first_n, last_n;
  float first_mult, last_mult;
};
// Pooling works on blocks of whole chunks of one prompt,
// pool_block_tokens(C) = C * max(1, floor(256 / C)) tokens each.
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
size_t select_ws(int B, int total_chunks);
hipError_t launch_select(int mode, double param, const SelectTable &t, const float *chunk_scores,
                         uint8_t *keep, int32_t *n_kept, void *ws, hipStream_t st);

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
