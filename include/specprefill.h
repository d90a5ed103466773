/*
 * libspecprefill: token-importance hot path of Speculative Prefill on
 * AMD Instinct MI355X (gfx950).
 *
 * A small draft model's lookahead queries attend over the whole prompt; the
 * attention they pay to each prompt token decides which 32-token chunks of the
 * prompt the large model prefills. Four calls, one per stage, run on a
 * caller-supplied HIP stream:
 *
 *   sp_score_attention  Q, K            -> importance[token]
 *   sp_pool_chunk       importance      -> token_scores[token], chunk_scores[chunk]
 *   sp_select_chunks    chunk_scores    -> keep[chunk], n_kept_chunks[prompt]
 *   sp_gather_kept      keep, token ids -> kept ids + original positions
 *   sp_pool_select_gather   the three calls above as one
 *   sp_break_even       host-side estimate: is sparse prefill worth running?
 * and the standalone tool's window and legacy-selection steps:
 *   sp_window_plan, sp_stitch_windows, sp_select_legacy
 *
 * Sources (web pages on SpecPrefill):
 *   [G]  "SpecPrefill — Implementation Guide": How It Works (Core Algorithm,
 *        Attention Capture, Token Importance, Chunk Selection, Sparse
 *        Prefill); v3 Improvements 1-2; v3.1 Optimizations & Bug Fixes 5;
 *        Configuration Reference; Implementation Details (Key Functions).
 *   [PR] "Speculative prefill" (llama.cpp pull request 27692): Approach,
 *        steps 1-4; Failure Mode Analysis & Operational Limits.
 *
 * Conventions for every call:
 *   - Ownership: the caller owns every buffer. The library allocates and
 *     frees nothing and keeps no pointer after a call returns. Work is
 *     enqueued on `stream` (a hipStream_t; NULL = the default stream), so
 *     the caller keeps inputs, outputs and the workspace alive until the
 *     stream reaches that point.
 *   - Memory: pointers named "host" are read during the call only; every
 *     other buffer pointer is device memory.
 *   - Errors: arguments are checked before anything is enqueued. A bad
 *     argument returns SP_ERR_INVALID_ARGUMENT, a valid but unsupported shape
 *     SP_ERR_UNSUPPORTED, a short workspace SP_ERR_WORKSPACE_TOO_SMALL; in each
 *     case nothing was launched. SP_ERR_DEVICE reports a failed launch.
 *     Faults during execution surface at the caller's next synchronisation.
 *   - Thread safety: calls on different streams with different workspaces
 *     may run concurrently (the global state is an atomic call counter and a
 *     per-device attribute cache). The library prints nothing.
 *   - Batches: B prompts, prompt b has N_b = token_offsets[b+1] -
 *     token_offsets[b] >= 1 tokens; per-token arrays are packed over the
 *     batch ([sum_b N_b]), per-chunk arrays likewise ([sum_b ceil(N_b / C)],
 *     prompt b's chunks first at sum_{b' < b} ceil(N_b' / C)).
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef SPECPREFILL_H
#define SPECPREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SP_ABI_VERSION 3
#define SP_MAX_PROMPTS 128          /* prompts per batch */
#define SP_MAX_CHUNKS_PER_PROMPT 16384

typedef enum {
  SP_OK = 0,
  SP_ERR_INVALID_ARGUMENT = 1,
  SP_ERR_UNSUPPORTED = 2,
  SP_ERR_WORKSPACE_TOO_SMALL = 3,
  SP_ERR_DEVICE = 4
} sp_status;

/* Element types of Q and K. SP_DTYPE_BF16_FP8K: Q bf16, K fp8 e4m3 codes
 * (OCP E4M3FN: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, max 448) with one fp32 scale per (layer, KV head): the key
 * value is k_scales[layer * n_kv_heads + kv_head] * code (a quantised draft
 * K cache: the [PR] discussion runs the draft model's K cache in an 8-bit
 * type through the draft KV-type options). */
typedef enum { SP_DTYPE_F32 = 0, SP_DTYPE_BF16 = 1, SP_DTYPE_BF16_FP8K = 2 } sp_dtype;

typedef enum { SP_SELECT_TOP_P = 0, SP_SELECT_MASS = 1 } sp_select_mode;

/* Scoring kernel choice: AUTO picks the fastest one that supports the shape:
 * the two-pass kernels for batches of at most 14336 keys (prompt tokens plus
 * lookahead) and wherever the single pass does not apply, else the single
 * pass. */
typedef enum {
  SP_SCORE_AUTO = 0,
  SP_SCORE_TWO_PASS = 1,   /* stats pass, then a recompute pass: K read twice */
  SP_SCORE_STREAM = 2      /* one persistent pass: K read once */
} sp_score_algo;

/* A batch of prompts. token_offsets is HOST memory, [n_prompts + 1],
 * token_offsets[0] == 0, strictly increasing. */
typedef struct {
  int32_t n_prompts;               /* 1 .. SP_MAX_PROMPTS */
  const int64_t *token_offsets;    /* host */
} sp_batch;

/* Draft attention shape ([G] Attention Capture; [PR] Approach steps 1-2).
 * n_lookahead (L) queries per prompt sit at positions N_b .. N_b + L - 1.
 * With prefill_row = 1 ([G] Full Source Code: the capture during the
 * prefill keeps the prompt's last row, and the importance averages it with
 * the lookahead rows) there are S = L + 1 query steps at positions
 * N_b - 1 .. N_b + L - 1; step 0 is the prompt's last token and sees only
 * the prompt. Without it S = L. */
typedef struct {
  int32_t n_layers;     /* attention layers that give scores, >= 1 */
  int32_t n_q_heads;    /* Hq >= 1 */
  int32_t n_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0; G = Hq / Hkv */
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t n_lookahead;  /* L >= 0 lookahead keys and steps; S >= 1; S * G <= 32 */
  int32_t dtype;        /* sp_dtype of Q and K */
  float scale;          /* logit scale, usually 1 / sqrt(d) */
  int32_t algo;         /* sp_score_algo */
  const float *k_scales; /* host, [n_layers * n_kv_heads], finite and > 0:
                            SP_DTYPE_BF16_FP8K only (n_layers * n_kv_heads
                            <= 128); NULL otherwise */
  int32_t prefill_row;  /* 0 or 1: step 0 is the prompt's last row */
  int32_t row_pool;     /* 0 or 1: off. Odd W in 3..33: pool-before-max, see
                           sp_score_attention; two-pass kernels, bf16 or f32 K */
} sp_attn_desc;

/* Smoothing, normalisation, boosts and chunking ([PR] Approach step 3;
 * [G] v3 item 2 and v3.1 item 5; [G] Configuration Reference defaults:
 * W 13, C 32, first 64 x1.5, last 128 x1.3). */
typedef struct {
  int32_t pool_window;       /* W: odd, >= 1 */
  int32_t chunk_size;        /* C: 1 .. 1024 */
  int32_t normalize;         /* 0/1: min-max scale each prompt's scores to [0, 1] */
  int32_t boost_first_n;     /* >= 0 */
  float boost_first_mult;    /* > 0; 1.0 = off */
  int32_t boost_last_n;      /* >= 0 */
  float boost_last_mult;     /* > 0; 1.0 = off */
} sp_pool_desc;

int sp_abi_version(void);
const char *sp_status_string(int status);

/* Workspace sizes (bytes, device memory) each call needs for this batch;
 * the result is written to *bytes. Alignment: 256 bytes (at least 16).
 * The selection needs none: sp_select_workspace_bytes writes 0 for every
 * valid batch (it checks the batch and chunk size like the call) and is
 * kept so that callers size every stage the same way. */
sp_status sp_score_workspace_bytes(const sp_attn_desc *desc, const sp_batch *batch,
                                   size_t *bytes);
sp_status sp_pool_workspace_bytes(const sp_pool_desc *desc, const sp_batch *batch,
                                  size_t *bytes);
sp_status sp_select_workspace_bytes(const sp_batch *batch, int32_t chunk_size, size_t *bytes);
sp_status sp_gather_workspace_bytes(const sp_batch *batch, int32_t chunk_size, size_t *bytes);

/*
 * Token importance ([G] Token Importance; [PR] Approach steps 1-3).
 * For every prompt b, layer l, step j and query head h, the softmax row of
 * query (b, l, j, h) over the keys it sees (keys 0 .. N_b - pre + j, causal,
 * pre = prefill_row: the prompt keys and the lookahead keys up to its own),
 * with logits scale * <q, k> against the key head h / G. Only the prompt
 * columns go forward ([G] capture callback).
 *   importance[b][k] = (1/S) * sum_j max_{l, h} p[b][l][j][h][k],  k < N_b
 * Pool-before-max (row_pool = W > 1; [PR] Approach step 3 lists the
 * smoothing before the max over heads and layers): each row's prompt
 * columns are first replaced by their centred W-key means over the prompt
 * keys inside the window (divided by that count),
 *   importance[b][k] = (1/S) * sum_j max_{l, h} pool_W(p[b][l][j][h])[k];
 * the caller then pools no more (sp_pool_chunk with pool_window 1).
 *
 *   q:  [B][n_layers][S][Hq][d] of dtype (bf16 for SP_DTYPE_BF16_FP8K),
 *       contiguous; S = L + prefill_row, step 0 the prefill row if any.
 *   k:  [n_layers][sum_b (N_b + L)][Hkv][d] of dtype (one byte per code for
 *       SP_DTYPE_BF16_FP8K, whose logits are scale * k_scales[l * Hkv + g] *
 *       <q, code>; single-pass kernel only), contiguous; prompt b's
 *       key rows start at token_offsets[b] + b * L: its N_b prompt keys, then
 *       its L lookahead keys.
 *   importance: [sum_b N_b] fp32 out.
 *   ws: device workspace of at least sp_score_workspace_bytes() bytes. Zero-fill
 *       it once before its first use (e.g. hipMemsetAsync) and leave it alone
 *       between calls; it then serves any sequence of calls with the same
 *       n_layers and n_kv_heads, whatever the batch or algorithm. Calls that
 *       share a workspace must not overlap in time.
 *   The single-pass kernel runs one block per compute unit and needs all of
 *   them resident together; the call checks the device's compute units
 *   before launching, and no other work should hold them meanwhile. Blocks
 *   exchange partial results through the workspace in slots that carry the
 *   posting call's tag, so nothing needs clearing between calls and a failed
 *   call leaves nothing a later one could take for its own.
 *   A block waits at most 2 s for another one (the SP_SCORE_WAIT_US
 *   environment variable, read at each call, sets another budget in
 *   microseconds), then finishes without hanging the device and marks the
 *   call as failed (importance is then not valid); sp_score_status()
 *   reports it. The workspace stays usable for the next call.
 */
sp_status sp_score_attention(const sp_attn_desc *desc, const sp_batch *batch, const void *q,
                             const void *k, float *importance, void *ws, size_t ws_bytes,
                             void *stream);

/* sp_score_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, kernels and results; the
 * workspace is instead a 48 MiB scratch array inside the library, one copy
 * per GPU, held until the process ends. The call allocates nothing.
 *   Returns SP_ERR_WORKSPACE_TOO_SMALL if the call needs more than 48 MiB:
 *   the single pass needs 256 B + 384 KiB per (layer, KV head) pair (up to
 *   127 pairs); the two-pass kernels (short batches under
 *   SP_SCORE_AUTO, SP_SCORE_TWO_PASS, pool-before-max) need
 *   sp_score_workspace_bytes(). SP_ERR_DEVICE if the scratch's address
 *   cannot be read on the current device.
 *   Every call on a GPU shares that GPU's scratch and finds it as the last
 *   call left it (nothing in it needs clearing): calls that overlap in time
 *   on one GPU, on any streams, race. Timed-out waits (see
 *   sp_score_status) are not reported for this variant. */
sp_status sp_score_attention_noalloc(const sp_attn_desc *desc, const sp_batch *batch,
                                     const void *q, const void *k, float *importance,
                                     void *stream);

/* What sp_score_attention would run for this descriptor and batch on the
 * current device, without running it: *kernel = SP_SCORE_STREAM (the
 * single pass) or SP_SCORE_TWO_PASS, by the same rule the call applies;
 * *n_launches = the single pass's kernel launches (a batch is split where
 * its prompts need more streaming blocks than the device has compute
 * units), 1 for the two-pass kernels; prompt_launch (HOST, [n_prompts], or
 * NULL) receives each prompt's launch. Returns the status the call would
 * return for these arguments (SP_ERR_UNSUPPORTED where the single pass is
 * demanded and does not take the shape). Host arithmetic and device
 * attribute queries only; nothing is enqueued. */
sp_status sp_score_plan(const sp_attn_desc *desc, const sp_batch *batch, int32_t *kernel,
                        int32_t *n_launches, int32_t *prompt_launch);

/* Whether the latest sp_score_attention (or sp_pool_select_gather) call on
 * this workspace completed: *status_host = 0 if so (or if there was none), 1
 * if a wait timed out and the results it wrote are not valid. Synchronises
 * `stream`. */
sp_status sp_score_status(const void *ws, int32_t *status_host, void *stream);

/*
 * Token and chunk scores ([PR] Approach step 3; [G] v3.1 item 5, v3 item 2,
 * Chunk Selection). Per prompt: centred average pooling of width W over the
 * positions inside the prompt; if normalize, min-max scaling to [0, 1] (a
 * prompt whose max - min <= 1e-6 * max gets 1.0 everywhere); then the boost
 * multipliers (both apply where the two ranges overlap); then the mean of
 * each C-token chunk over the tokens it holds.
 *
 *   importance:   [sum N_b] fp32 in.
 *   token_scores: [sum N_b] fp32 out (the boosted scores), or NULL.
 *   chunk_scores: [sum ceil(N_b / C)] fp32 out.
 */
sp_status sp_pool_chunk(const sp_pool_desc *desc, const sp_batch *batch, const float *importance,
                        float *token_scores, float *chunk_scores, void *ws, size_t ws_bytes,
                        void *stream);

/*
 * Chunk selection per prompt ([PR] Approach step 4; [G] v3 item 1).
 * The final chunk (prompt boundary) is always kept; the other chunks are
 * visited by score, highest first, ties to the lower index.
 *   SP_SELECT_TOP_P: param = p in (0, 1]; keeps kc = max(1, min(nc,
 *     ceil(p * nc - 1e-9))) chunks (computed in double), the final one
 *     included.
 *   SP_SELECT_MASS: param = mass in (0, 1]; keeps the final chunk, then
 *     chunks in visiting order while the kept score sum is below
 *     mass * (sum of all chunk scores); the chunk that reaches it is kept.
 * Arithmetic: scores are ranked and summed as 64-bit fixed point scaled to
 * the prompt's largest score (resolution 2^-48 of it; exact, order-free
 * sums), ranked on the top 32 bits of that value: scores closer than 2^-32
 * of the largest count as equal and go by index.
 *
 *   chunk_scores:  [sum nc_b] fp32 in (finite, >= 0).
 *   keep:          [sum nc_b] uint8 out (0/1).
 *   n_kept_chunks: [B] int32 out.
 *   ws, ws_bytes: not used (the selection needs no workspace; may be NULL).
 */
sp_status sp_select_chunks(int32_t mode, double param, const sp_batch *batch, int32_t chunk_size,
                           const float *chunk_scores, uint8_t *keep, int32_t *n_kept_chunks,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * Kept-token compaction ([G] Sparse Prefill; [PR] Approach step 4): the
 * first token (BOS) and every token of a kept chunk, ascending, with its
 * token id and its original position inside the prompt (gaps preserved).
 *
 *   keep:         [sum nc_b] uint8 in.
 *   token_ids:    [sum N_b] int32 in.
 *   kept_ids:     [sum N_b] int32 out (capacity); prompt b's kept tokens at
 *                 kept_offsets[b] .. kept_offsets[b+1].
 *   kept_pos:     [sum N_b] int32 out, same layout.
 *   kept_offsets: [B + 1] int64 out.
 */
sp_status sp_gather_kept(const sp_batch *batch, int32_t chunk_size, const uint8_t *keep,
                         const int32_t *token_ids, int32_t *kept_ids, int32_t *kept_pos,
                         int64_t *kept_offsets, void *ws, size_t ws_bytes, void *stream);

/*
 * sp_pool_chunk, sp_select_chunks and sp_gather_kept in one call, with the
 * same arguments and bit-identical results ([PR] Approach steps 3-4; [G]
 * v3.1 item 5, v3 items 1-2, Chunk Selection, Sparse Prefill). On the device
 * the three stages run in one of three forms (sp_pool_select_gather_form
 * tells which):
 *   SP_POST_DIE: one launch in which each chip die (XCD) runs the whole
 *     batch with one block per compute unit (ranges of whole chunks of one
 *     prompt, up to 8192 tokens and 1024 chunks each; at most 32 prompts and
 *     one range per CU of a die); blocks hand each other values only within
 *     their die, and every block finds its prompt's selection cutoff itself;
 *   SP_POST_GRID: one launch of at most one block per compute unit over the
 *     whole device (blocks of up to 2048 tokens and 64 chunks), the blocks
 *     handing each other min/max, chunk scores and kept counts;
 *   SP_POST_SEPARATE: the three stages' own kernels, for batches that need
 *     more blocks than that.
 *
 *   pool:         as sp_pool_chunk (its chunk_size is C).
 *   mode, param:  as sp_select_chunks.
 *   importance:   [sum N_b] fp32 in.
 *   token_ids:    [sum N_b] int32 in.
 *   token_scores: [sum N_b] fp32 out, or NULL.
 *   chunk_scores, keep, n_kept_chunks: out, as sp_pool_chunk and
 *                 sp_select_chunks.
 *   kept_ids, kept_pos, kept_offsets: out, as sp_gather_kept.
 *   ws: device workspace (16-byte aligned) of at least
 *       sp_pool_select_gather_workspace_bytes() bytes; it starts with the
 *       same status header as the scoring workspace, and never needs
 *       clearing.
 * Waits between blocks are bounded like the scoring call's (2 s, or
 * SP_SCORE_WAIT_US): a call whose wait ran out writes no kept ids or
 * positions and sp_score_status() on its workspace reports 1.
 */
sp_status sp_pool_select_gather_workspace_bytes(const sp_pool_desc *pool, const sp_batch *batch,
                                                size_t *bytes);
sp_status sp_pool_select_gather(const sp_pool_desc *pool, int32_t mode, double param,
                                const sp_batch *batch, const float *importance,
                                const int32_t *token_ids, float *token_scores,
                                float *chunk_scores, uint8_t *keep, int32_t *n_kept_chunks,
                                int32_t *kept_ids, int32_t *kept_pos, int64_t *kept_offsets,
                                void *ws, size_t ws_bytes, void *stream);
/* The tokens per block of the one-launch form of sp_pool_select_gather for
 * this batch on the current device, or 0 when the call runs the separate
 * kernels. Host arithmetic and device attribute queries only. */
sp_status sp_pool_select_gather_plan(const sp_pool_desc *pool, const sp_batch *batch,
                                     int32_t *block_tokens);
/* The form of sp_pool_select_gather for this batch on the current device
 * (*form: SP_POST_DIE, SP_POST_GRID or SP_POST_SEPARATE) and its tokens per
 * block (0 for SP_POST_SEPARATE). Host arithmetic and device attribute
 * queries only. */
#define SP_POST_SEPARATE 0
#define SP_POST_GRID 1
#define SP_POST_DIE 2
sp_status sp_pool_select_gather_form(const sp_pool_desc *pool, const sp_batch *batch,
                                     int32_t *form, int32_t *block_tokens);

/*
 * Standalone-tool semantics ([G] Sliding Window and its worked example,
 * v3.1 Optimizations & Bug Fixes items 6-7, Sliding Window Loop (v3.1 —
 * fixed), Configuration Reference: SP_CHUNK, SP_KEEP_PCT, SP_MAX_KEEP; the
 * chunk-selection and main-loop parts of [G] Full Source Code). The tool
 * scores a long prompt window by window, each window a prompt of its own for
 * the draft model; the windows go to sp_score_attention as one batch.
 */

/* Window plan (host arithmetic, no device work): windows start at 0, stride,
 * 2 stride, ... and span min(window, n_tokens - start) tokens. A window is the
 * last one when it reaches the end of the prompt or when the next start would
 * (start + stride >= n_tokens); it keeps all of its tokens' scores, every
 * other window the first `stride` ones. Writes the number of windows to
 * *n_windows and, when it fits in `capacity`, the windows to starts, lengths
 * and keep_lengths (host arrays). A count above capacity, or NULL arrays,
 * returns SP_ERR_INVALID_ARGUMENT with *n_windows still set: call with
 * capacity 0 and NULL arrays to learn the size. Also SP_ERR_INVALID_ARGUMENT
 * for n_tokens < 1 (or >= 2^30), window < 1, stride outside 1..window. */
sp_status sp_window_plan(int64_t n_tokens, int32_t window, int32_t stride, int32_t capacity,
                         int64_t *starts, int32_t *lengths, int32_t *keep_lengths,
                         int32_t *n_windows);

/* Prompt scores from window scores: token t gets the mean of the scores that
 * the windows holding t in their kept range give it (window w's token
 * t - starts[w]), and 1.0 if no window does.
 *   windows: the window batch (window w = prompt w, host offsets).
 *   starts, keep_lengths: host, [n_windows]; keep_lengths[w] <= window
 *     length, starts[w] + keep_lengths[w] <= n_tokens.
 *   window_importance: [sum of window lengths] fp32 in (sp_score_attention
 *     on the window batch).
 *   scores: [n_tokens] fp32 out. */
sp_status sp_stitch_windows(const sp_batch *windows, const int64_t *starts,
                            const int32_t *keep_lengths, int64_t n_tokens,
                            const float *window_importance, float *scores, void *stream);

/* Legacy chunk rule of the tool, per prompt, plus its cap on tokens sent to
 * the target. With eff_min = min(min_tokens, max(4, N / 10)): if
 * keep_pct >= 1 or N <= eff_min every token is kept. Otherwise, with
 * kc = max(1, ceil(nc * keep_pct)) computed in single precision, a chunk is
 * kept when fewer than kc chunk scores of the prompt are strictly larger
 * (its score reaches the kc-th largest: ties are all kept); tokens 0-3 and,
 * for N > 4, the last two are kept too; while fewer than eff_min tokens are
 * kept, the remaining tokens are added in index order. The kept tokens, in
 * ascending order, are then capped: above max_keep of them, every step-th
 * one is kept (step = count / max_keep, integer division) up to max_keep,
 * the last slot taking the final kept token.
 *   chunk_scores: [sum nc_b] fp32 in (e.g. sp_pool_chunk with pool_window 1).
 *   token_ids: [sum N_b] int32 in.
 *   kept_ids, kept_pos: [sum N_b] int32 out (capacity), prompt b's at
 *     kept_offsets[b] .. kept_offsets[b + 1].
 *   kept_offsets: [B + 1] int64 out.
 *   ws: device workspace of sp_select_legacy_workspace_bytes() bytes. */
sp_status sp_select_legacy_workspace_bytes(const sp_batch *batch, int32_t chunk_size,
                                           size_t *bytes);
sp_status sp_select_legacy(const sp_batch *batch, int32_t chunk_size, float keep_pct,
                           int32_t min_tokens, int32_t max_keep, const float *chunk_scores,
                           const int32_t *token_ids, int32_t *kept_ids, int32_t *kept_pos,
                           int64_t *kept_offsets, void *ws, size_t ws_bytes, void *stream);

/*
 * Break-even gate ([G] v3 Improvements item 4 and Configuration Reference:
 * SP_BREAK_EVEN, SP_SPEC_THROUGHPUT, SP_BREAK_EVEN_SAFETY). Host arithmetic,
 * no device work; a caller runs it before scoring, with the number of tokens
 * it expects to keep. In double precision:
 *   scoring_time = n_tokens / spec_tps
 *   saved_time   = (n_tokens - n_kept) / target_tps
 *   *run = 0 (skip sparse prefill) if saved_time < scoring_time * safety,
 *          else 1.
 * A value <= 0 selects the guide's default: spec_tps 600, target_tps 270,
 * safety 1.2.
 *   n_tokens >= 1, 0 <= n_kept <= n_tokens; arguments finite; run non-NULL.
 */
sp_status sp_break_even(int64_t n_tokens, int64_t n_kept, double spec_tps, double target_tps,
                        double safety, int32_t *run);

#ifdef __cplusplus
}
#endif

#endif /* SPECPREFILL_H */
