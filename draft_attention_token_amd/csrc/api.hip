// C ABI of libspecprefill: argument checks, per-prompt tables, workspace
// layout and launches. Every check runs before anything is enqueued.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "sp_internal.h"

namespace sp {

uint32_t reserve_tags(int n) {
  static std::atomic<uint32_t> next{1u};
  for (;;) {
    const uint32_t base = next.fetch_add((uint32_t)n);
    // Tag 0 marks a never-written slot: skip a range that wraps through it.
    if (base != 0u && (uint32_t)(base + (uint32_t)(n - 1)) >= base) return base;
  }
}

}  // namespace sp

using namespace sp;

namespace {

// Largest batch (keys: prompt tokens plus lookahead) that AUTO scores with the
// two-pass kernels.
constexpr int64_t kAutoTwoPassKeys = 14336;

constexpr int64_t kMaxTotalTokens = (int64_t)1 << 30;   // keeps int32 token offsets safe

// Checks a batch; on success fills N (per prompt) and the token total.
sp_status check_batch(const sp_batch *batch, int64_t *total) {
  if (!batch || !batch->token_offsets) return SP_ERR_INVALID_ARGUMENT;
  if (batch->n_prompts < 1) return SP_ERR_INVALID_ARGUMENT;
  if (batch->n_prompts > SP_MAX_PROMPTS) return SP_ERR_UNSUPPORTED;
  const int64_t *off = batch->token_offsets;
  if (off[0] != 0) return SP_ERR_INVALID_ARGUMENT;
  for (int b = 0; b < batch->n_prompts; ++b)
    if (off[b + 1] <= off[b]) return SP_ERR_INVALID_ARGUMENT;
  if (off[batch->n_prompts] >= kMaxTotalTokens) return SP_ERR_UNSUPPORTED;
  *total = off[batch->n_prompts];
  return SP_OK;
}

// Table with unit_off[b] = prefix of ceil((N_b + extra) / per) and tok_off.
SegTable make_table(const sp_batch *batch, int extra, int per, int L) {
  SegTable t;
  memset(&t, 0, sizeof(t));
  t.B = batch->n_prompts;
  t.L = L;
  t.unit_off[0] = 0;
  for (int b = 0; b < t.B; ++b) {
    const int64_t n = batch->token_offsets[b + 1] - batch->token_offsets[b];
    t.unit_off[b + 1] = t.unit_off[b] + (int32_t)((n + extra + per - 1) / per);
    t.tok_off[b] = (int32_t)batch->token_offsets[b];
  }
  t.tok_off[t.B] = (int32_t)batch->token_offsets[t.B];
  return t;
}

PoolTable make_pool_table(const sp_batch *batch, int C) {
  const int TB = pool_block_tokens(C);
  PoolTable t;
  memset(&t, 0, sizeof(t));
  t.B = batch->n_prompts;
  for (int b = 0; b < t.B; ++b) {
    const int64_t n = batch->token_offsets[b + 1] - batch->token_offsets[b];
    t.blk_off[b + 1] = t.blk_off[b] + (int32_t)((n + TB - 1) / TB);
    t.chunk_off[b + 1] = t.chunk_off[b] + (int32_t)((n + C - 1) / C);
    t.tok_off[b] = (int32_t)batch->token_offsets[b];
  }
  t.tok_off[t.B] = (int32_t)batch->token_offsets[t.B];
  return t;
}

sp_status check_attn(const sp_attn_desc *d, AttnShape *s) {
  if (!d) return SP_ERR_INVALID_ARGUMENT;
  if (d->n_layers < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->n_lookahead < 0)
    return SP_ERR_INVALID_ARGUMENT;
  if (d->prefill_row != 0 && d->prefill_row != 1) return SP_ERR_INVALID_ARGUMENT;
  if (d->n_lookahead + d->prefill_row < 1) return SP_ERR_INVALID_ARGUMENT;
  if (d->row_pool < 0 || (d->row_pool > 1 && d->row_pool % 2 == 0)) return SP_ERR_INVALID_ARGUMENT;
  if (d->row_pool > kMaxRowPool) return SP_ERR_UNSUPPORTED;
  if (d->n_q_heads % d->n_kv_heads != 0) return SP_ERR_INVALID_ARGUMENT;
  if (d->dtype != SP_DTYPE_F32 && d->dtype != SP_DTYPE_BF16 && d->dtype != SP_DTYPE_BF16_FP8K)
    return SP_ERR_INVALID_ARGUMENT;
  if (!(isfinite(d->scale))) return SP_ERR_INVALID_ARGUMENT;
  if (d->algo < SP_SCORE_AUTO || d->algo > SP_SCORE_STREAM) return SP_ERR_INVALID_ARGUMENT;
  if (d->head_dim != 64 && d->head_dim != 128) return SP_ERR_UNSUPPORTED;
  const int G = d->n_q_heads / d->n_kv_heads;
  if ((int64_t)(d->n_lookahead + d->prefill_row) * G > kRows) return SP_ERR_UNSUPPORTED;
  if (d->row_pool > 1 && (d->algo == SP_SCORE_STREAM || d->dtype == SP_DTYPE_BF16_FP8K))
    return SP_ERR_UNSUPPORTED;                                      // two-pass kernels only
  if (d->dtype == SP_DTYPE_BF16_FP8K) {
    if (d->algo == SP_SCORE_TWO_PASS) return SP_ERR_UNSUPPORTED;   // single-pass only
    if ((int64_t)d->n_layers * d->n_kv_heads > kMaxScaledProblems) return SP_ERR_UNSUPPORTED;
  }
  s->n_layers = d->n_layers;
  s->Hq = d->n_q_heads;
  s->Hkv = d->n_kv_heads;
  s->d = d->head_dim;
  s->L = d->n_lookahead + d->prefill_row;
  s->G = G;
  s->La = d->n_lookahead;
  s->pre = d->prefill_row;
  s->row_pool = d->row_pool > 1 ? d->row_pool : 1;
  s->scale_log2 = d->scale * kLog2e;
  s->dtype = d->dtype;
  return SP_OK;
}

sp_status check_pool(const sp_pool_desc *d, PoolParams *p) {
  if (!d) return SP_ERR_INVALID_ARGUMENT;
  if (d->pool_window < 1 || d->pool_window % 2 == 0) return SP_ERR_INVALID_ARGUMENT;
  if (d->pool_window > kMaxPoolWindow) return SP_ERR_UNSUPPORTED;
  if (d->chunk_size < 1) return SP_ERR_INVALID_ARGUMENT;
  if (d->chunk_size > 1024) return SP_ERR_UNSUPPORTED;
  if (d->normalize != 0 && d->normalize != 1) return SP_ERR_INVALID_ARGUMENT;
  if (d->boost_first_n < 0 || d->boost_last_n < 0) return SP_ERR_INVALID_ARGUMENT;
  if (!(d->boost_first_mult > 0.f) || !(d->boost_last_mult > 0.f) ||
      !isfinite(d->boost_first_mult) || !isfinite(d->boost_last_mult))
    return SP_ERR_INVALID_ARGUMENT;
  p->W = d->pool_window;
  p->C = d->chunk_size;
  p->normalize = d->normalize;
  p->first_n = d->boost_first_n;
  p->last_n = d->boost_last_n;
  p->first_mult = d->boost_first_mult;
  p->last_mult = d->boost_last_mult;
  return SP_OK;
}

sp_status check_chunks(const sp_batch *batch, int32_t C, int *max_nc) {
  if (C < 1) return SP_ERR_INVALID_ARGUMENT;
  if (C > 1024) return SP_ERR_UNSUPPORTED;
  int m = 0;
  for (int b = 0; b < batch->n_prompts; ++b) {
    const int64_t n = batch->token_offsets[b + 1] - batch->token_offsets[b];
    const int64_t nc = (n + C - 1) / C;
    if (nc > SP_MAX_CHUNKS_PER_PROMPT) return SP_ERR_UNSUPPORTED;
    if (nc > m) m = (int)nc;
  }
  *max_nc = m;
  return SP_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool check_select_args(int32_t mode, double param) {
  return (mode == SP_SELECT_TOP_P || mode == SP_SELECT_MASS) && param > 0.0 && param <= 1.0;
}

// Selection tables: chunk prefix, rank-kernel blocks and the top-p budget
// kc = clamp(ceil(p * nc), 1, nc) of each prompt.
SelectTable make_select_table(const SegTable &chunks, double param) {
  SelectTable t;
  memset(&t, 0, sizeof(t));
  t.B = chunks.B;
  for (int b = 0; b < chunks.B; ++b) {
    const int nc = chunks.unit_off[b + 1] - chunks.unit_off[b];
    t.chunk_off[b + 1] = chunks.unit_off[b + 1];
    t.blk_off[b + 1] = t.blk_off[b] + select_rank_blocks(nc);
    int64_t v = (int64_t)ceil(param * (double)nc - 1e-9);
    if (v > nc) v = nc;
    if (v < 1) v = 1;
    t.kc[b] = (int32_t)v;
  }
  return t;
}

// Tokens per block of the fused post-scoring launch: the smallest multiple of
// the pool group (pool_block_tokens(C); at most kPostMaxTB tokens and
// kPostMaxChunks chunks) whose blocks number at most max_blocks, with at
// most kPostMaxGroups groups in a prompt; 0 when there is none.
int post_block_tokens(const sp_batch *batch, int C, int max_blocks) {
  const int GT = pool_block_tokens(C);
  for (int b = 0; b < batch->n_prompts; ++b)
    if ((batch->token_offsets[b + 1] - batch->token_offsets[b] + GT - 1) / GT > kPostMaxGroups)
      return 0;
  const int64_t total = batch->token_offsets[batch->n_prompts];
  int per = (int)std::max<int64_t>(1, total / ((int64_t)std::max(1, max_blocks) * GT));
  for (; (int64_t)per * GT <= kPostMaxTB && (int64_t)per * GT / C <= kPostMaxChunks; ++per) {
    const int64_t TB = (int64_t)per * GT;
    int64_t G = 0;
    for (int b = 0; b < batch->n_prompts; ++b)
      G += (batch->token_offsets[b + 1] - batch->token_offsets[b] + TB - 1) / TB;
    if (G <= max_blocks) return (int)TB;
  }
  return 0;
}

// Tokens per range of the die-local launch: the smallest multiple of the
// pool group (at most kDieMaxTB tokens and kDieMaxChunks chunks) whose
// ranges number at most `ranges` (the CUs of one die), for batches of at
// most kDieMaxPrompts prompts with at most kPostMaxGroups groups each; 0
// when there is none.
int post_die_block_tokens(const sp_batch *batch, int C, int ranges) {
  const int B = batch->n_prompts;
  if (ranges <= 0 || B > kDieMaxPrompts || B > ranges) return 0;
  const int GT = pool_block_tokens(C);
  for (int b = 0; b < B; ++b)
    if ((batch->token_offsets[b + 1] - batch->token_offsets[b] + GT - 1) / GT > kPostMaxGroups)
      return 0;
  const int64_t total = batch->token_offsets[B];
  int per = (int)std::max<int64_t>(1, total / ((int64_t)ranges * GT));
  for (; (int64_t)per * GT <= kDieMaxTB && (int64_t)per * GT / C <= kDieMaxChunks; ++per) {
    const int64_t TB = (int64_t)per * GT;
    int64_t n = 0;
    for (int b = 0; b < B; ++b)
      n += (batch->token_offsets[b + 1] - batch->token_offsets[b] + TB - 1) / TB;
    if (n <= ranges) return (int)TB;
  }
  return 0;
}

// The form sp_pool_select_gather takes for a batch on the current device,
// and its tokens per block (range).
int post_form(const sp_batch *batch, int C, int32_t *block_tokens) {
  int tb = post_die_block_tokens(batch, C, post_die_ranges());
  if (tb > 0) {
    *block_tokens = tb;
    return SP_POST_DIE;
  }
  tb = post_block_tokens(batch, C, post_max_blocks());
  *block_tokens = tb;
  return tb > 0 ? SP_POST_GRID : SP_POST_SEPARATE;
}

// Workspace of sp_pool_select_gather: the status header, then the slots of
// either one-launch form or the separate kernels' workspaces (pool, gather).
size_t post_split_bytes(const PoolTable &pt, const SegTable &chunks) {
  return align_up(pool_ws(pt.B, pt.blk_off[pt.B])) + gather_ws(chunks.B, chunks.unit_off[chunks.B]);
}
size_t post_ws_bytes(const PoolTable &pt, const SegTable &chunks) {
  // The pool table's blocks are the pool groups.
  const int NC = chunks.unit_off[chunks.B], G = pt.blk_off[pt.B];
  return kStatusBytes + std::max({post_slot_bytes(NC, G), post_die_slot_bytes(chunks.B, NC, G),
                                  post_split_bytes(pt, chunks)});
}

// Scoring workspace: header, single-pass slots, two-pass region (one layout
// for every algorithm, so calls with different algorithms can share it).
size_t score_ws_bytes(const AttnShape &s, const SegTable &tiles) {
  return kStatusBytes + score_stream_slot_bytes(s) +
         score_two_pass_region_bytes(s, tiles.B, tiles.unit_off[tiles.B]);
}

sp_status launched(hipError_t e) { return e == hipSuccess ? SP_OK : SP_ERR_DEVICE; }

// The scoring kernel a call runs: the single pass for SP_SCORE_STREAM, fp8 K,
// and AUTO on batches of more than kAutoTwoPassKeys keys, when it takes the
// shape; else the two-pass kernels. AUTO gives short batches to the two-pass
// kernels: there the single pass is bound by its per-problem hand-offs,
// while the two passes run every (tile, problem) pair at once.
sp_status choose_kernel(const sp_attn_desc *desc, const AttnShape &s, const SegTable &tiles,
                        bool *stream) {
  const bool f8 = s.dtype == SP_DTYPE_BF16_FP8K;
  if ((desc->algo == SP_SCORE_STREAM || f8) && !score_stream_supported(s))
    return SP_ERR_UNSUPPORTED;
  const int64_t total_keys = (int64_t)tiles.tok_off[tiles.B] + (int64_t)tiles.B * s.La;
  const bool short_batch = total_keys <= kAutoTwoPassKeys;
  *stream = desc->algo == SP_SCORE_STREAM || f8 || (desc->algo == SP_SCORE_AUTO && !short_batch);
  if (*stream && !score_stream_supported(s)) *stream = false;   // AUTO on another shape
  return SP_OK;
}

// A validated sp_score_attention call: its shape, key tiles, fp8 scales
// and the kernel it takes.
struct ScoreCall {
  AttnShape s;
  SegTable tiles;
  KScales ks;
  bool use_stream = false;   // the single pass, if the plan takes the batch
  bool must_stream = false;  // no two-pass fallback (SP_SCORE_STREAM or fp8 K)
};

sp_status prepare_score(const sp_attn_desc *desc, const sp_batch *batch, const void *q,
                        const void *k, float *importance, ScoreCall *c) {
  int64_t total;
  sp_status st = check_attn(desc, &c->s);
  if (st != SP_OK) return st;
  if ((st = check_batch(batch, &total)) != SP_OK) return st;
  if (!q || !k || !importance) return SP_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k)) return SP_ERR_INVALID_ARGUMENT;
  const bool f8 = c->s.dtype == SP_DTYPE_BF16_FP8K;
  if (f8) {
    if (!desc->k_scales) return SP_ERR_INVALID_ARGUMENT;
    const int P = c->s.n_layers * c->s.Hkv;
    for (int x = 0; x < P; ++x) {
      const float v = desc->k_scales[x];
      if (!(v > 0.f) || !isfinite(v)) return SP_ERR_INVALID_ARGUMENT;
      c->ks.v[x] = v;
    }
  }
  c->tiles = make_table(batch, c->s.La, kTile, c->s.La);
  c->must_stream = desc->algo == SP_SCORE_STREAM || f8;
  return choose_kernel(desc, c->s, c->tiles, &c->use_stream);
}

// Scratch of sp_score_attention_noalloc: the scoring workspace of calls that
// may not allocate, one copy per GPU, held until the process ends. Host code
// uses only the device addresses hipGetSymbolAddress returns for it.
constexpr size_t kNoAllocBytes = size_t(48) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

// The scratch's address on the current device, taken once per device with
// that device current (each GPU holds its own copy at its own address).
void *scratch_on_current_device() {
  constexpr int kMaxDevices = 64;
  static void *addr[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

int sp_abi_version(void) { return SP_ABI_VERSION; }

const char *sp_status_string(int status) {
  switch (status) {
    case SP_OK: return "ok";
    case SP_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SP_ERR_UNSUPPORTED: return "unsupported shape or size";
    case SP_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SP_ERR_DEVICE: return "device launch failed";
    default: return "unknown status";
  }
}

sp_status sp_score_workspace_bytes(const sp_attn_desc *desc, const sp_batch *batch,
                                   size_t *bytes) {
  if (!bytes) return SP_ERR_INVALID_ARGUMENT;
  AttnShape s;
  int64_t total;
  sp_status st = check_attn(desc, &s);
  if (st != SP_OK) return st;
  if ((st = check_batch(batch, &total)) != SP_OK) return st;
  const SegTable tiles = make_table(batch, s.La, kTile, s.La);
  *bytes = score_ws_bytes(s, tiles);
  return SP_OK;
}


sp_status sp_score_plan(const sp_attn_desc *desc, const sp_batch *batch, int32_t *kernel,
                        int32_t *n_launches, int32_t *prompt_launch) {
  if (!kernel || !n_launches) return SP_ERR_INVALID_ARGUMENT;
  AttnShape s;
  int64_t total;
  sp_status st = check_attn(desc, &s);
  if (st != SP_OK) return st;
  if ((st = check_batch(batch, &total)) != SP_OK) return st;
  const SegTable tiles = make_table(batch, s.La, kTile, s.La);
  bool stream = false;
  if ((st = choose_kernel(desc, s, tiles, &stream)) != SP_OK) return st;
  if (stream) {
    int launches = 0;
    if (score_stream_plan(s, tiles, &launches, prompt_launch)) {
      *kernel = SP_SCORE_STREAM;
      *n_launches = launches;
      return SP_OK;
    }
    if (desc->algo == SP_SCORE_STREAM || s.dtype == SP_DTYPE_BF16_FP8K) return SP_ERR_UNSUPPORTED;
  }
  *kernel = SP_SCORE_TWO_PASS;
  *n_launches = 1;
  if (prompt_launch)
    for (int b = 0; b < batch->n_prompts; ++b) prompt_launch[b] = 0;
  return SP_OK;
}

sp_status sp_score_attention(const sp_attn_desc *desc, const sp_batch *batch, const void *q,
                             const void *k, float *importance, void *ws, size_t ws_bytes,
                             void *stream) {
  ScoreCall c;
  sp_status st = prepare_score(desc, batch, q, k, importance, &c);
  if (st != SP_OK) return st;
  if (!aligned16(ws)) return SP_ERR_INVALID_ARGUMENT;
  if (!ws || ws_bytes < score_ws_bytes(c.s, c.tiles)) return SP_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (c.use_stream) {
    bool supported = false;
    const hipError_t e = launch_score_stream(c.s, c.tiles, q, k, c.ks, importance, ws, hs, &supported);
    if (supported) return launched(e);
    if (c.must_stream) return SP_ERR_UNSUPPORTED;
  }
  char *region = reinterpret_cast<char *>(ws) + kStatusBytes + score_stream_slot_bytes(c.s);
  return launched(launch_score_two_pass(c.s, c.tiles, c.tiles.unit_off[c.tiles.B], q, k, importance,
                                        reinterpret_cast<uint32_t *>(ws), region, hs));
}

sp_status sp_score_attention_noalloc(const sp_attn_desc *desc, const sp_batch *batch,
                                     const void *q, const void *k, float *importance,
                                     void *stream) {
  ScoreCall c;
  sp_status st = prepare_score(desc, batch, q, k, importance, &c);
  if (st != SP_OK) return st;
  // The scratch takes sp_score_attention's workspace layout (header,
  // single-pass slots, two-pass region), so neither kernel's data lands on
  // the other's slots; the single pass needs only the first two parts.
  int launches = 0;
  const bool stream_plan = c.use_stream && score_stream_plan(c.s, c.tiles, &launches, nullptr);
  if (c.use_stream && !stream_plan && c.must_stream) return SP_ERR_UNSUPPORTED;
  const size_t need = stream_plan ? kStatusBytes + score_stream_slot_bytes(c.s)
                                  : score_ws_bytes(c.s, c.tiles);
  if (need > kNoAllocBytes) return SP_ERR_WORKSPACE_TOO_SMALL;
  char *ws = reinterpret_cast<char *>(scratch_on_current_device());
  if (!ws) return SP_ERR_DEVICE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (stream_plan) {
    bool supported = false;
    const hipError_t e = launch_score_stream(c.s, c.tiles, q, k, c.ks, importance, ws, hs, &supported);
    if (supported) return launched(e);
    // (The plan took the batch a moment ago; should it not now, the two
    // passes run only if their region fits too.)
    if (c.must_stream || score_ws_bytes(c.s, c.tiles) > kNoAllocBytes) return SP_ERR_UNSUPPORTED;
  }
  return launched(launch_score_two_pass(c.s, c.tiles, c.tiles.unit_off[c.tiles.B], q, k, importance,
                                        reinterpret_cast<uint32_t *>(ws),
                                        ws + kStatusBytes + score_stream_slot_bytes(c.s), hs));
}

sp_status sp_score_status(const void *ws, int32_t *status_host, void *stream) {
  if (!ws || !status_host) return SP_ERR_INVALID_ARGUMENT;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  uint32_t hdr[2] = {0u, 0u};
  if (hipMemcpyAsync(hdr, ws, sizeof(hdr), hipMemcpyDeviceToHost, hs) != hipSuccess ||
      hipStreamSynchronize(hs) != hipSuccess)
    return SP_ERR_DEVICE;
  *status_host = (hdr[1] != 0u && hdr[0] == hdr[1]) ? 1 : 0;
  return SP_OK;
}

sp_status sp_pool_workspace_bytes(const sp_pool_desc *desc, const sp_batch *batch,
                                  size_t *bytes) {
  if (!bytes) return SP_ERR_INVALID_ARGUMENT;
  PoolParams p;
  int64_t total;
  sp_status st = check_pool(desc, &p);
  if (st != SP_OK) return st;
  if ((st = check_batch(batch, &total)) != SP_OK) return st;
  const PoolTable t = make_pool_table(batch, p.C);
  *bytes = pool_ws(t.B, t.blk_off[t.B]);
  return SP_OK;
}

sp_status sp_pool_chunk(const sp_pool_desc *desc, const sp_batch *batch, const float *importance,
                        float *token_scores, float *chunk_scores, void *ws, size_t ws_bytes,
                        void *stream) {
  PoolParams p;
  int64_t total;
  int max_nc;
  sp_status st = check_pool(desc, &p);
  if (st != SP_OK) return st;
  if ((st = check_batch(batch, &total)) != SP_OK) return st;
  if ((st = check_chunks(batch, p.C, &max_nc)) != SP_OK) return st;
  if (!importance || !chunk_scores) return SP_ERR_INVALID_ARGUMENT;
  const PoolTable t = make_pool_table(batch, p.C);
  const size_t need = pool_ws(t.B, t.blk_off[t.B]);
  if (ws_bytes < need || !ws) return SP_ERR_WORKSPACE_TOO_SMALL;
  return launched(launch_pool_chunk(p, t, importance, token_scores, chunk_scores, ws,
                                    reinterpret_cast<hipStream_t>(stream)));
}

sp_status sp_select_workspace_bytes(const sp_batch *batch, int32_t chunk_size, size_t *bytes) {
  if (!bytes) return SP_ERR_INVALID_ARGUMENT;
  int64_t total;
  int max_nc;
  sp_status st = check_batch(batch, &total);
  if (st != SP_OK) return st;
  if ((st = check_chunks(batch, chunk_size, &max_nc)) != SP_OK) return st;
  *bytes = 0;   // the selection needs no workspace
  return SP_OK;
}

sp_status sp_select_chunks(int32_t mode, double param, const sp_batch *batch, int32_t chunk_size,
                           const float *chunk_scores, uint8_t *keep, int32_t *n_kept_chunks,
                           void *ws, size_t ws_bytes, void *stream) {
  int64_t total;
  int max_nc;
  if (!check_select_args(mode, param)) return SP_ERR_INVALID_ARGUMENT;
  sp_status st = check_batch(batch, &total);
  if (st != SP_OK) return st;
  if ((st = check_chunks(batch, chunk_size, &max_nc)) != SP_OK) return st;
  if (!chunk_scores || !keep || !n_kept_chunks) return SP_ERR_INVALID_ARGUMENT;
  (void)ws;   // none needed (see sp_select_workspace_bytes)
  (void)ws_bytes;
  const SegTable chunks = make_table(batch, 0, chunk_size, 0);
  const SelectTable t = make_select_table(chunks, param);
  return launched(launch_select(mode, param, t, chunk_scores, keep, n_kept_chunks,
                                reinterpret_cast<hipStream_t>(stream)));
}

sp_status sp_gather_workspace_bytes(const sp_batch *batch, int32_t chunk_size, size_t *bytes) {
  if (!bytes) return SP_ERR_INVALID_ARGUMENT;
  int64_t total;
  int max_nc;
  sp_status st = check_batch(batch, &total);
  if (st != SP_OK) return st;
  if ((st = check_chunks(batch, chunk_size, &max_nc)) != SP_OK) return st;
  const SegTable chunks = make_table(batch, 0, chunk_size, 0);
  *bytes = gather_ws(chunks.B, chunks.unit_off[chunks.B]);
  return SP_OK;
}

sp_status sp_gather_kept(const sp_batch *batch, int32_t chunk_size, const uint8_t *keep,
                         const int32_t *token_ids, int32_t *kept_ids, int32_t *kept_pos,
                         int64_t *kept_offsets, void *ws, size_t ws_bytes, void *stream) {
  int64_t total;
  int max_nc;
  sp_status st = check_batch(batch, &total);
  if (st != SP_OK) return st;
  if ((st = check_chunks(batch, chunk_size, &max_nc)) != SP_OK) return st;
  if (!keep || !token_ids || !kept_ids || !kept_pos || !kept_offsets)
    return SP_ERR_INVALID_ARGUMENT;
  const SegTable chunks = make_table(batch, 0, chunk_size, 0);
  const SegTable blocks = make_table(batch, 0, kGatherBlockTokens, 0);
  const size_t need = gather_ws(chunks.B, chunks.unit_off[chunks.B]);
  if (ws_bytes < need || !ws) return SP_ERR_WORKSPACE_TOO_SMALL;
  return launched(launch_gather(chunks, blocks, blocks.unit_off[blocks.B], chunk_size, keep,
                                token_ids, kept_ids, kept_pos, kept_offsets, ws,
                                reinterpret_cast<hipStream_t>(stream)));
}

sp_status sp_pool_select_gather_workspace_bytes(const sp_pool_desc *pool, const sp_batch *batch,
                                                size_t *bytes) {
  if (!bytes) return SP_ERR_INVALID_ARGUMENT;
  PoolParams p;
  int64_t total;
  int max_nc;
  sp_status st = check_pool(pool, &p);
  if (st != SP_OK) return st;
  if ((st = check_batch(batch, &total)) != SP_OK) return st;
  if ((st = check_chunks(batch, p.C, &max_nc)) != SP_OK) return st;
  *bytes = post_ws_bytes(make_pool_table(batch, p.C), make_table(batch, 0, p.C, 0));
  return SP_OK;
}

sp_status sp_pool_select_gather(const sp_pool_desc *pool, int32_t mode, double param,
                                const sp_batch *batch, const float *importance,
                                const int32_t *token_ids, float *token_scores,
                                float *chunk_scores, uint8_t *keep, int32_t *n_kept_chunks,
                                int32_t *kept_ids, int32_t *kept_pos, int64_t *kept_offsets,
                                void *ws, size_t ws_bytes, void *stream) {
  PoolParams p;
  int64_t total;
  int max_nc;
  if (!check_select_args(mode, param)) return SP_ERR_INVALID_ARGUMENT;
  sp_status st = check_pool(pool, &p);
  if (st != SP_OK) return st;
  if ((st = check_batch(batch, &total)) != SP_OK) return st;
  if ((st = check_chunks(batch, p.C, &max_nc)) != SP_OK) return st;
  if (!importance || !token_ids || !chunk_scores || !keep || !n_kept_chunks || !kept_ids ||
      !kept_pos || !kept_offsets)
    return SP_ERR_INVALID_ARGUMENT;
  if (!aligned16(ws)) return SP_ERR_INVALID_ARGUMENT;
  const PoolTable pt = make_pool_table(batch, p.C);
  const SegTable chunks = make_table(batch, 0, p.C, 0);
  if (!ws || ws_bytes < post_ws_bytes(pt, chunks)) return SP_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const SelectTable sel = make_select_table(chunks, param);
  int32_t TB = 0;
  const int form = post_form(batch, p.C, &TB);
  if (form == SP_POST_DIE) {
    DieTable t;
    memset(&t, 0, sizeof(t));
    t.B = batch->n_prompts;
    t.TB = TB;
    t.GT = pool_block_tokens(p.C);
    t.by_gt = fast_div((uint32_t)t.GT);
    t.by_c = fast_div((uint32_t)p.C);
    t.by_cpg = fast_div((uint32_t)(t.GT / p.C));
    t.by_runs = fast_div((uint32_t)((p.C + 7) / 8));
    for (int b = 0; b < t.B; ++b) {
      const int64_t n = batch->token_offsets[b + 1] - batch->token_offsets[b];
      t.rng_off[b + 1] = t.rng_off[b] + (int32_t)((n + TB - 1) / TB);
      t.chunk_off[b + 1] = chunks.unit_off[b + 1];
      t.grp_off[b + 1] = pt.blk_off[b + 1];
      t.tok_off[b] = chunks.tok_off[b];
      t.kc[b] = sel.kc[b];
    }
    t.tok_off[t.B] = chunks.tok_off[t.B];
    t.NR = t.rng_off[t.B];
    return launched(launch_post_die(mode, param, p, t, importance, token_ids, token_scores,
                                    chunk_scores, keep, n_kept_chunks, kept_ids, kept_pos,
                                    kept_offsets, ws, hs));
  }
  if (form == SP_POST_GRID) {
    PostTable t;
    memset(&t, 0, sizeof(t));
    t.B = batch->n_prompts;
    t.TB = TB;
    t.GT = pool_block_tokens(p.C);
    for (int b = 0; b < t.B; ++b) {
      const int64_t n = batch->token_offsets[b + 1] - batch->token_offsets[b];
      t.blk_off[b + 1] = t.blk_off[b] + (int32_t)((n + TB - 1) / TB);
      t.chunk_off[b + 1] = chunks.unit_off[b + 1];
      t.grp_off[b + 1] = pt.blk_off[b + 1];
      t.tok_off[b] = chunks.tok_off[b];
      t.kc[b] = sel.kc[b];
    }
    t.tok_off[t.B] = chunks.tok_off[t.B];
    t.G = t.blk_off[t.B];
    return launched(launch_post(mode, param, p, t, importance, token_ids, token_scores,
                                chunk_scores, keep, n_kept_chunks, kept_ids, kept_pos,
                                kept_offsets, ws, hs));
  }
  // The separate kernels, on the regions after the header.
  char *pool_region = reinterpret_cast<char *>(ws) + kStatusBytes;
  char *gather_region = pool_region + align_up(pool_ws(pt.B, pt.blk_off[pt.B]));
  const SegTable blocks = make_table(batch, 0, kGatherBlockTokens, 0);
  hipError_t e = launch_stamp(ws, hs);
  if (e == hipSuccess)
    e = launch_pool_chunk(p, pt, importance, token_scores, chunk_scores, pool_region, hs);
  if (e == hipSuccess)
    e = launch_select(mode, param, sel, chunk_scores, keep, n_kept_chunks, hs);
  if (e == hipSuccess)
    e = launch_gather(chunks, blocks, blocks.unit_off[blocks.B], p.C, keep, token_ids, kept_ids,
                      kept_pos, kept_offsets, gather_region, hs);
  return launched(e);
}

sp_status sp_pool_select_gather_plan(const sp_pool_desc *pool, const sp_batch *batch, int32_t *block_tokens) {
  PoolParams p;
  int64_t total;
  int max_nc;
  if (!block_tokens) return SP_ERR_INVALID_ARGUMENT;
  sp_status st = check_pool(pool, &p);
  if (st != SP_OK) return st;
  if ((st = check_batch(batch, &total)) != SP_OK) return st;
  if ((st = check_chunks(batch, p.C, &max_nc)) != SP_OK) return st;
  post_form(batch, p.C, block_tokens);
  return SP_OK;
}

sp_status sp_pool_select_gather_form(const sp_pool_desc *pool, const sp_batch *batch,
                                     int32_t *form, int32_t *block_tokens) {
  PoolParams p;
  int64_t total;
  int max_nc;
  if (!form || !block_tokens) return SP_ERR_INVALID_ARGUMENT;
  sp_status st = check_pool(pool, &p);
  if (st != SP_OK) return st;
  if ((st = check_batch(batch, &total)) != SP_OK) return st;
  if ((st = check_chunks(batch, p.C, &max_nc)) != SP_OK) return st;
  *form = post_form(batch, p.C, block_tokens);
  return SP_OK;
}

sp_status sp_window_plan(int64_t n_tokens, int32_t window, int32_t stride, int32_t capacity,
                         int64_t *starts, int32_t *lengths, int32_t *keep_lengths,
                         int32_t *n_windows) {
  if (!n_windows) return SP_ERR_INVALID_ARGUMENT;
  *n_windows = 0;
  if (n_tokens < 1 || n_tokens >= kMaxTotalTokens || window < 1 || stride < 1 || stride > window)
    return SP_ERR_INVALID_ARGUMENT;
  // Windows start at 0, stride, 2 stride, ...; the first one that reaches the
  // end of the prompt, or whose successor would start at or past it, is the
  // last, and it keeps all of its tokens (the others keep their first stride).
  int64_t count = 0;
  for (int64_t pos = 0;; pos += stride) {
    const int64_t end = pos + window < n_tokens ? pos + window : n_tokens;
    const bool last = end >= n_tokens || pos + stride >= n_tokens;
    if (count < capacity && starts && lengths && keep_lengths) {
      starts[count] = pos;
      lengths[count] = (int32_t)(end - pos);
      keep_lengths[count] = (int32_t)(last ? end - pos : stride);
    }
    ++count;
    if (last) break;
  }
  *n_windows = (int32_t)count;
  if (count > capacity || !starts || !lengths || !keep_lengths) return SP_ERR_INVALID_ARGUMENT;
  return SP_OK;
}

sp_status sp_stitch_windows(const sp_batch *windows, const int64_t *starts,
                            const int32_t *keep_lengths, int64_t n_tokens,
                            const float *window_importance, float *scores, void *stream) {
  int64_t total;
  sp_status st = check_batch(windows, &total);
  if (st != SP_OK) return st;
  if (!starts || !keep_lengths || !window_importance || !scores) return SP_ERR_INVALID_ARGUMENT;
  if (n_tokens < 1 || n_tokens >= kMaxTotalTokens) return SP_ERR_INVALID_ARGUMENT;
  StitchTable t;
  memset(&t, 0, sizeof(t));
  t.n_windows = windows->n_prompts;
  for (int w = 0; w < t.n_windows; ++w) {
    const int64_t len = windows->token_offsets[w + 1] - windows->token_offsets[w];
    if (starts[w] < 0 || keep_lengths[w] < 0 || keep_lengths[w] > len ||
        starts[w] + keep_lengths[w] > n_tokens)
      return SP_ERR_INVALID_ARGUMENT;
    t.start[w] = (int32_t)starts[w];
    t.keep[w] = keep_lengths[w];
    t.win_off[w] = (int32_t)windows->token_offsets[w];
  }
  return launched(launch_stitch(t, (int32_t)n_tokens, window_importance, scores,
                                reinterpret_cast<hipStream_t>(stream)));
}

sp_status sp_select_legacy_workspace_bytes(const sp_batch *batch, int32_t chunk_size,
                                           size_t *bytes) {
  if (!bytes) return SP_ERR_INVALID_ARGUMENT;
  int64_t total;
  int max_nc;
  sp_status st = check_batch(batch, &total);
  if (st != SP_OK) return st;
  if ((st = check_chunks(batch, chunk_size, &max_nc)) != SP_OK) return st;
  const SegTable chunks = make_table(batch, 0, chunk_size, 0);
  *bytes = legacy_ws(chunks.B, chunks.unit_off[chunks.B], nullptr).bytes;
  return SP_OK;
}

sp_status sp_select_legacy(const sp_batch *batch, int32_t chunk_size, float keep_pct,
                           int32_t min_tokens, int32_t max_keep, const float *chunk_scores,
                           const int32_t *token_ids, int32_t *kept_ids, int32_t *kept_pos,
                           int64_t *kept_offsets, void *ws, size_t ws_bytes, void *stream) {
  int64_t total;
  int max_nc;
  sp_status st = check_batch(batch, &total);
  if (st != SP_OK) return st;
  if ((st = check_chunks(batch, chunk_size, &max_nc)) != SP_OK) return st;
  if (!(keep_pct > 0.f) || !isfinite(keep_pct) || min_tokens < 0 || max_keep < 1)
    return SP_ERR_INVALID_ARGUMENT;
  if (!chunk_scores || !token_ids || !kept_ids || !kept_pos || !kept_offsets)
    return SP_ERR_INVALID_ARGUMENT;
  const SegTable chunks = make_table(batch, 0, chunk_size, 0);
  if (!ws || ws_bytes < legacy_ws(chunks.B, chunks.unit_off[chunks.B], nullptr).bytes)
    return SP_ERR_WORKSPACE_TOO_SMALL;
  LegacyTable t;
  memset(&t, 0, sizeof(t));
  t.B = chunks.B;
  t.C = chunk_size;
  t.max_keep = max_keep;
  for (int b = 0; b < t.B; ++b) {
    const int32_t n = chunks.tok_off[b + 1] - chunks.tok_off[b];
    const int32_t nc = chunks.unit_off[b + 1] - chunks.unit_off[b];
    t.tok_off[b] = chunks.tok_off[b];
    t.chunk_off[b] = chunks.unit_off[b];
    t.blk_off[b + 1] = t.blk_off[b] + legacy_rank_blocks(nc);
    t.wblk_off[b + 1] = t.wblk_off[b] + legacy_write_blocks(n);
    // Effective minimum min(min_tokens, max(4, n / 10)); a prompt no longer
    // than it, or keep_pct >= 1, keeps every chunk and needs no fill.
    const int32_t eff = std::min(min_tokens, std::max(4, n / 10));
    if (keep_pct >= 1.f || n <= eff) {
      t.kc[b] = nc;
      t.eff_min[b] = 0;
    } else {
      const float prod = (float)nc * keep_pct;   // single precision, as the tool reads it
      t.kc[b] = std::min(nc, std::max(1, (int32_t)ceilf(prod)));
      t.eff_min[b] = eff;
    }
  }
  t.tok_off[t.B] = chunks.tok_off[t.B];
  t.chunk_off[t.B] = chunks.unit_off[t.B];
  return launched(launch_legacy(t, chunk_scores, token_ids, ws, kept_ids, kept_pos, kept_offsets,
                                reinterpret_cast<hipStream_t>(stream)));
}

sp_status sp_break_even(int64_t n_tokens, int64_t n_kept, double spec_tps, double target_tps,
                        double safety, int32_t *run) {
  if (!run || n_tokens < 1 || n_kept < 0 || n_kept > n_tokens) return SP_ERR_INVALID_ARGUMENT;
  if (!isfinite(spec_tps) || !isfinite(target_tps) || !isfinite(safety))
    return SP_ERR_INVALID_ARGUMENT;
  const double spec = spec_tps > 0.0 ? spec_tps : 600.0;      // speculator tokens/s
  const double target = target_tps > 0.0 ? target_tps : 270.0;  // target-model tokens/s
  const double margin = safety > 0.0 ? safety : 1.2;
  const double scoring_time = (double)n_tokens / spec;
  const double saved_time = (double)(n_tokens - n_kept) / target;
  *run = saved_time < scoring_time * margin ? 0 : 1;
  return SP_OK;
}

}  // extern "C"
