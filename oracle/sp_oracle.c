/*
 * Plain CPU oracle of the SpecPrefill token-importance path.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously correct
 * definition the HIP library is checked against. Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg load it; the library never does.
 * It shares no code, header, table or helper with the HIP path.
 *
 * Arithmetic is fp64 throughout, on the caller's fp32 input values (bf16
 * inputs arrive widened to fp32, which is exact). Loops follow the
 * definitions directly: no blocking, no fusion, no reordering.
 *
 * Sources (web pages on SpecPrefill):
 *  [G]  "SpecPrefill — Implementation Guide" (sliding-specprefill project):
 *       How It Works (Core Algorithm, Attention Capture, Token Importance,
 *       Chunk Selection, Sparse Prefill); v3 Improvements (1. Cumulative
 *       Attention Mass Selection, 2. Structural Token Boosting); v3.1
 *       Optimizations & Bug Fixes (5. Score Normalization); Configuration
 *       Reference (v3 Variables); Full Source Code (compute_imp,
 *       select_chunks, capture callback).
 *  [PR] "Speculative prefill", llama.cpp pull request 27692: Approach
 *       (steps 1-4); Failure Mode Analysis & Operational Limits (kept-token
 *       tables).
 *
 * Readings where the pages are silent or disagree are marked READING.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC sp_oracle.c -o libsp_oracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_version(void) { return 1; }

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Softmax row of one lookahead query over its visible keys.
 *
 * [PR] Approach step 2 and [G] Attention Capture: the draft's post-softmax
 * attention rows (kq_soft_max) are read for each lookahead query. Query j of
 * prompt b sits at position N_b + j and is causal, so it sees keys
 * 0 .. N_b + j (N_b prompt keys and its own and earlier lookahead keys):
 *     s_k = scale * <Q[b][l][j][h], K[l][key0 + k][h / G]>
 *     p_k = exp(s_k - max s) / sum_k' exp(s_k' - max s)
 * Prefill row (pre = 1; [G] Full Source Code, the capture callback and the
 * window loop): the last row of the prompt's own prefill is captured too and
 * counts as one more step, in front of the lookahead ones. Then S = L + 1
 * steps, step j sits at position N_b - 1 + j, and step 0 sees exactly the
 * prompt's keys. In general step j (0 <= j < L + pre) sees keys
 * 0 .. N_b - pre + j.
 * Writes p[0 .. N_b - pre + j]. Returns 0, or -1 on bad args.
 *
 *   q: [B][layers][L + pre][Hq][d]   k: [layers][sum_b (N_b + L)][Hkv][d]
 *   tok_off: [B + 1]; prompt b's key rows start at tok_off[b] + b * L.
 *   k_scales: NULL, or [layers][Hkv]: a quantised K cache (the [PR]
 *   discussion runs the draft's K cache in an 8-bit type) holds codes, and
 *   the key is k_scales[l][g] * code, so
 *     s_k = scale * <Q, k_scales[l][h / G] * K_code> = scale * k_scales[l][h / G] * <Q, K_code>.
 */
int oracle_softmax_row(int B, const int64_t *tok_off, int n_layers, int Hq,
                       int Hkv, int d, int L, int pre, double scale, const float *q,
                       const float *k, int b, int l, int j, int h, double *p,
                       const double *k_scales) {
  const int S = L + pre;
  if (b < 0 || b >= B || l < 0 || l >= n_layers || j < 0 || j >= S || h < 0 ||
      h >= Hq || Hkv <= 0 || Hq % Hkv != 0 || L < 0 || pre < 0 || pre > 1)
    return -1;
  const int G = Hq / Hkv;
  const int64_t total_keys = tok_off[B] + (int64_t)B * L;
  const int64_t N = tok_off[b + 1] - tok_off[b];
  const int64_t key0 = tok_off[b] + (int64_t)b * L;
  const float *qrow = q + ((((int64_t)b * n_layers + l) * S + j) * Hq + h) * d;
  const int64_t nvis = N - pre + j + 1;
  const double ks = k_scales ? k_scales[(int64_t)l * Hkv + h / G] : 1.0;
  double m = -INFINITY;
  for (int64_t kk = 0; kk < nvis; kk++) {
    const float *krow = k + (((int64_t)l * total_keys + key0 + kk) * Hkv + h / G) * d;
    double s = 0.0;
    for (int e = 0; e < d; e++) s += (double)qrow[e] * (double)krow[e];
    s *= scale * ks;
    p[kk] = s;
    if (s > m) m = s;
  }
  double z = 0.0;
  for (int64_t kk = 0; kk < nvis; kk++) z += exp(p[kk] - m);
  for (int64_t kk = 0; kk < nvis; kk++) p[kk] = exp(p[kk] - m) / z;
  return 0;
}

/*
 * Centred average pool of width W (odd) over in[0 .. n): each output is the
 * mean of the inputs within (W - 1) / 2 positions that lie inside [0, n)
 * (divided by their count). [PR] Approach step 3; the edge rule is the one
 * oracle_pool_chunk states.
 */
static void box_mean(int64_t n, const double *in, int W, double *out) {
  const int64_t r = (W - 1) / 2;
  for (int64_t t = 0; t < n; t++) {
    const int64_t lo = t - r < 0 ? 0 : t - r;
    const int64_t hi = t + r > n - 1 ? n - 1 : t + r;
    double s = 0.0;
    for (int64_t i = lo; i <= hi; i++) s += in[i];
    out[t] = s / (double)(hi - lo + 1);
  }
}

/*
 * Token importance of every prompt token (steps: softmax rows, max over
 * heads, max over layers, mean over the S = L + pre steps; pre: see
 * oracle_softmax_row).
 *
 * Pool-before-max (row_pool = W > 1): [PR] Approach step 3 lists the
 * smoothing before the max over heads and layers. In that order each
 * probability row's prompt columns are pooled (box_mean, width W) before
 * they enter the max; row_pool = 1 leaves the rows as they are (the pooling
 * then happens once, later, on the importance: oracle_pool_chunk).
 *
 * [G] Token Importance and compute_imp: for each lookahead step, take the
 * maximum attention probability over all heads, then over all attention
 * layers; then average the per-step values over the steps.
 * [G] capture callback: only the first N columns (the prompt keys) of each
 * row are read, although each row is normalised over every key it sees.
 *
 *   imp[tok_off[b] + k] = (1/S) * sum_j max_{l, h} p[b][l][j][h][k],  k < N_b
 *
 * Parallel over (prompt, step, layer) triples when built with OpenMP; each
 * takes its heads' max in a row of its own and merges it into the (prompt,
 * step) row under a lock. Maxima are exact in any order and the mean over
 * steps runs afterwards in step order, so the result does not depend on the
 * thread count.
 * nthreads <= 0 uses the OpenMP default. Returns 0, or -1 on bad args.
 */
int oracle_importance(int B, const int64_t *tok_off, int n_layers, int Hq,
                      int Hkv, int d, int L, int pre, int row_pool, double scale,
                      const float *q, const float *k, double *imp, int nthreads,
                      const double *k_scales) {
  if (B <= 0 || n_layers <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 ||
      d <= 0 || L < 0 || pre < 0 || pre > 1 || L + pre <= 0 || row_pool < 1 ||
      row_pool % 2 == 0)
    return -1;
  const int S = L + pre;
  const int64_t total_tok = tok_off[B];
  int64_t max_n = 0;
  for (int b = 0; b < B; b++) {
    const int64_t n = tok_off[b + 1] - tok_off[b];
    if (n <= 0) return -1;
    if (n > max_n) max_n = n;
  }
  /* stepmax[b][j][k] lives at stepmax[(tok_off[b] * S) + j * N_b + k]. */
  double *stepmax = (double *)malloc(sizeof(double) * (size_t)(total_tok * S));
  if (!stepmax) return -1;
  for (int64_t i = 0; i < total_tok * S; i++) stepmax[i] = 0.0; /* probabilities are >= 0 */
  int err = 0;
  /* One task per (prompt, step, layer): its Hq rows, max into a private row,
   * then max into the (prompt, step) row under that row's lock. A max is
   * exact in any order, so the result does not depend on the thread count. */
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  omp_lock_t *locks = (omp_lock_t *)malloc(sizeof(omp_lock_t) * (size_t)(B * S));
  if (!locks) { free(stepmax); return -1; }
  for (int i = 0; i < B * S; i++) omp_init_lock(&locks[i]);
#pragma omp parallel for collapse(3) schedule(dynamic) num_threads(nthreads) reduction(| : err)
#endif
  for (int b = 0; b < B; b++) {
    for (int j = 0; j < S; j++) {
      for (int l = 0; l < n_layers; l++) {
        const int64_t N = tok_off[b + 1] - tok_off[b];
        double *sm = stepmax + tok_off[b] * S + (int64_t)j * N;
        double *p = (double *)malloc(sizeof(double) * (size_t)(N + L));
        double *pooled = (double *)malloc(sizeof(double) * (size_t)N);
        double *mine = (double *)malloc(sizeof(double) * (size_t)N);
        if (!p || !pooled || !mine) { free(p); free(pooled); free(mine); err |= 1; continue; }
        for (int64_t kk = 0; kk < N; kk++) mine[kk] = 0.0;
        for (int h = 0; h < Hq; h++) {
          oracle_softmax_row(B, tok_off, n_layers, Hq, Hkv, d, L, pre, scale, q, k,
                             b, l, j, h, p, k_scales);
          const double *row = p;
          if (row_pool > 1) {  /* the row's prompt columns only */
            box_mean(N, p, row_pool, pooled);
            row = pooled;
          }
          for (int64_t kk = 0; kk < N; kk++)  /* prompt columns only */
            if (row[kk] > mine[kk]) mine[kk] = row[kk];
        }
#ifdef _OPENMP
        omp_set_lock(&locks[b * S + j]);
#endif
        for (int64_t kk = 0; kk < N; kk++)
          if (mine[kk] > sm[kk]) sm[kk] = mine[kk];
#ifdef _OPENMP
        omp_unset_lock(&locks[b * S + j]);
#endif
        free(p);
        free(pooled);
        free(mine);
      }
    }
  }
#ifdef _OPENMP
  for (int i = 0; i < B * S; i++) omp_destroy_lock(&locks[i]);
  free(locks);
#endif
  if (!err) {
    for (int b = 0; b < B; b++) {
      const int64_t N = tok_off[b + 1] - tok_off[b];
      for (int64_t kk = 0; kk < N; kk++) {
        double acc = 0.0;
        for (int j = 0; j < S; j++) acc += stepmax[tok_off[b] * S + (int64_t)j * N + kk];
        imp[tok_off[b] + kk] = acc / S;
      }
    }
  }
  free(stepmax);
  return err ? -1 : 0;
}

/*
 * Token scores and chunk scores of one prompt of n tokens.
 *
 * 1. Smoothing, [PR] Approach step 3: 1-D average pooling with window W.
 *    READING: the window is centred (W odd, radius (W-1)/2) and averages only
 *    the positions inside the prompt (divide by the number present), so a
 *    constant signal stays constant at the edges.
 * 2. Normalisation, [G] v3.1 item 5: min-max scaling of the scores to [0, 1]
 *    before boosting and selection. READING: over this prompt's n pooled
 *    scores; if (max - min) <= 1e-6 * max the scores carry no signal and all
 *    become 1.0 (the pages' own no-signal value in compute_imp).
 * 3. Boosts, [G] v3 item 2 and Configuration Reference: the first first_n
 *    tokens are multiplied by first_mult and the last last_n by last_mult;
 *    a multiplier of 1.0 disables it. READING: where the two ranges overlap,
 *    both multipliers apply.
 * 4. Chunk means, [G] Chunk Selection and select_chunks: contiguous chunks of
 *    C tokens; a chunk's score is the mean over the tokens it holds (the last
 *    chunk may be shorter).
 *
 * token_scores: [n] (may be NULL); chunk_scores: [ceil(n / C)].
 * Returns 0, or -1 on bad args (n <= 0, W even or < 1, C < 1).
 */
int oracle_pool_chunk(int64_t n, const double *imp, int W, int C, int normalize,
                      int first_n, double first_mult, int last_n,
                      double last_mult, double *token_scores,
                      double *chunk_scores) {
  if (n <= 0 || W < 1 || W % 2 == 0 || C < 1) return -1;
  double *x = (double *)malloc(sizeof(double) * (size_t)n);
  if (!x) return -1;
  box_mean(n, imp, W, x);
  if (normalize) {
    double mn = x[0], mx = x[0];
    for (int64_t t = 1; t < n; t++) {
      if (x[t] < mn) mn = x[t];
      if (x[t] > mx) mx = x[t];
    }
    if (mx - mn <= 1e-6 * mx) {
      for (int64_t t = 0; t < n; t++) x[t] = 1.0;
    } else {
      for (int64_t t = 0; t < n; t++) x[t] = (x[t] - mn) / (mx - mn);
    }
  }
  for (int64_t t = 0; t < n; t++) {
    if (t < first_n) x[t] *= first_mult;
    if (t >= n - last_n) x[t] *= last_mult;
  }
  const int64_t nc = (n + C - 1) / C;
  for (int64_t c = 0; c < nc; c++) {
    const int64_t s0 = c * C, s1 = (c + 1) * C < n ? (c + 1) * C : n;
    double s = 0.0;
    for (int64_t t = s0; t < s1; t++) s += x[t];
    chunk_scores[c] = s / (double)(s1 - s0);
  }
  if (token_scores)
    for (int64_t t = 0; t < n; t++) token_scores[t] = x[t];
  free(x);
  return 0;
}

/* Chunk order used by both selection rules: higher score first, and among
 * equal scores the lower chunk index first ("ties by lower index"). Returns
 * nonzero when chunk a comes before chunk b. */
static int before(const double *cs, int64_t a, int64_t b) {
  if (cs[a] != cs[b]) return cs[a] > cs[b];
  return a < b;
}

/* The non-final chunks 0 .. nc-2 in selection order (simple insertion sort:
 * slow and obviously right). */
static int64_t *ranked_non_final(int64_t nc, const double *cs) {
  int64_t *ord = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nc > 1 ? nc - 1 : 1));
  if (!ord) return NULL;
  for (int64_t i = 0; i < nc - 1; i++) {
    int64_t pos = i;
    while (pos > 0 && before(cs, i, ord[pos - 1])) {
      ord[pos] = ord[pos - 1];
      pos--;
    }
    ord[pos] = i;
  }
  return ord;
}

/*
 * Number of chunks fixed top-p keeps: [PR] Approach step 4 keeps the top-p
 * fraction of chunks; [G] select_chunks rounds the chunk count up, with at
 * least one. READING (pinned by every kept-token count in [PR]'s stress
 * tables): kc = max(1, min(nc, ceil(p * nc - 1e-9))) in double, and the
 * always-kept final chunk counts inside kc. The 1e-9 guard stops a product
 * such as 0.08 * 25 that should be an integer from rounding up.
 */
int64_t oracle_top_p_count(int64_t nc, double p) {
  int64_t kc = (int64_t)ceil(p * (double)nc - 1e-9);
  if (kc > nc) kc = nc;
  if (kc < 1) kc = 1;
  return kc;
}

/*
 * Fixed top-p chunk selection ([PR] Approach step 4). The final chunk (the
 * prompt boundary) is always kept; the other kc - 1 slots go to the best
 * non-final chunks in selection order. keep: [nc] 0/1. Returns the number of
 * kept chunks, or -1 on bad args.
 */
int64_t oracle_select_top_p(int64_t nc, const double *cs, double p, uint8_t *keep) {
  if (nc <= 0 || !(p > 0.0) || p > 1.0) return -1;
  const int64_t kc = oracle_top_p_count(nc, p);
  int64_t *ord = ranked_non_final(nc, cs);
  if (!ord) return -1;
  memset(keep, 0, (size_t)nc);
  keep[nc - 1] = 1;
  for (int64_t i = 0; i < kc - 1; i++) keep[ord[i]] = 1;
  free(ord);
  return kc;
}

/*
 * Cumulative-mass chunk selection ([G] v3 item 1): walk the chunks from the
 * highest score down and keep them until the kept share of the total chunk
 * mass reaches the threshold. READING: the mass of a chunk is its score (the
 * chunk mean that ranks it); the always-kept final chunk is kept first and
 * its mass counts; "reaches" means >=, so the chunk whose mass crosses the
 * threshold is kept; the walk visits the non-final chunks in selection order.
 * Returns the number of kept chunks, or -1 on bad args.
 */
int64_t oracle_select_mass(int64_t nc, const double *cs, double mass, uint8_t *keep) {
  if (nc <= 0 || !(mass > 0.0) || mass > 1.0) return -1;
  double total = 0.0;
  for (int64_t i = 0; i < nc; i++) total += cs[i];
  const double target = mass * total;
  int64_t *ord = ranked_non_final(nc, cs);
  if (!ord) return -1;
  memset(keep, 0, (size_t)nc);
  keep[nc - 1] = 1;
  int64_t kept = 1;
  double cum = cs[nc - 1];
  for (int64_t i = 0; i < nc - 1 && cum < target; i++) {
    keep[ord[i]] = 1;
    cum += cs[ord[i]];
    kept++;
  }
  free(ord);
  return kept;
}

/*
 * Kept-token compaction ([G] Sparse Prefill; [PR] Approach step 4): the kept
 * tokens are the first token (BOS) and every token of a kept chunk, in
 * ascending order, each with its token id and its original position in the
 * prompt (positions keep their gaps). Returns the number written.
 */
int64_t oracle_gather(int64_t n, int C, const uint8_t *keep, const int32_t *ids,
                      int32_t *kept_ids, int32_t *kept_pos) {
  if (n <= 0 || C < 1) return -1;
  int64_t w = 0;
  for (int64_t t = 0; t < n; t++) {
    if (t == 0 || keep[t / C]) {
      kept_ids[w] = ids[t];
      kept_pos[w] = (int32_t)t;
      w++;
    }
  }
  return w;
}
