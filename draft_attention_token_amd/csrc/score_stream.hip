// Token importance, single-pass streaming form: K is read from HBM once.
//
// Method: "SpecPrefill — Implementation Guide", How It Works / Token
// Importance (max over heads, then layers, then mean over lookahead steps);
// "Speculative prefill" (llama.cpp pull request 27692), Approach steps 2-3.
// Query j of a prompt sits at position N + j and sees keys 0 .. N + j; only
// the N prompt columns receive importance.
//
// Design. A probability needs its row's log-sum-exp (lse) over every key the
// row sees, so no probability is final before all of K has been read. Rather
// than read K twice, the logits stay on chip and the lse arrives later:
//
//  * Persistent grid, one block per CU (a block's shared memory admits only
//    one per unit), all blocks resident at once. A block owns <= 18
//    contiguous 32-key tiles of one prompt for the whole kernel (prompt keys
//    and lookahead keys alike).
//  * The work is a sequence of problems (layer l, KV group g), each with
//    L * G <= 32 query rows (step j, head-in-group hh), padded to 32.
//  * Six compute waves per block, <= 3 tiles each. Per problem a wave
//    computes logits with 32x32x16 bf16 MFMA, K as the A operand (MFMA row =
//    key) and Q as the B operand (MFMA column = query row): a lane holds one
//    query row and 16 keys of each tile, so a row's max and sum over the
//    wave's keys reduce inside the lane plus one swap of wave halves. As
//    soon as a tile's MFMAs have consumed its K registers, the wave refills
//    them with the next problem's tile: the K stream never waits for
//    synchronisation. Statistics are accumulated tile by tile (online max,
//    rescaled sum); each tile's e = 2^(x - m) is relative to the running max
//    m at that tile, kept per tile.
//  * The last compute wave to finish a problem merges the six waves'
//    statistics into the block's partial base-2 lse of each row and posts
//    it to the workspace (one float per row) at once.
//  * Two control waves do the rest of the cross-block work, so no compute
//    wave ever waits on a load other than its own K (on this hardware a
//    wait on any load also waits on every load issued before it, which
//    would drain the K prefetch). They take alternate problems: for its
//    problem x a control wave stages Q(x + 1) (prefetched into its
//    registers), then reads every block's partials of x (plain loads,
//    shared through the L2 of its chip die), merges them in block order and
//    stages the row lse of x in LDS. Compute and control waves hand data
//    over through LDS flags rather than block barriers, so a slow
//    cross-block read only stalls the compute waves when they need its
//    result.
//  * The compute waves fold problem i - 2 while working on problem i: they
//    park e in LDS (two problem slots) and turn it into probabilities
//    p = e * 2^(m_tile - lse) once the lse is staged, kept as a running max
//    per (row, key) in registers (max over layers and KV groups).
//  * Finally: max over the G heads of a step (lanes of a group), mean over
//    the L steps (a butterfly across groups of lanes), store.
//
// Partial slots. A slot holding all-zero bits has not been posted (a posted
// value is never +0.0: it is stored as -0.0). A block that reads an empty
// slot (not posted yet, or a stale copy in its die's L2) reads it again with
// a load that bypasses the L2. Slots are left empty for the next launch:
// once a block has merged every block's partials of problem x, every block
// has finished reading the partials of problem x - 3 (a block posts x only
// after folding x - 2, which needs its merge of x - 2 and, before that, of
// x - 3), so the block clears its own slots of x - 3; the last block to
// finish clears the final three problems' slots of every block. A zero-filled
// workspace is therefore ready for the first launch and stays ready.
//
// Every wait is bounded (about 2 s); on time-out the kernel records it in the
// workspace header and runs to completion, so the grid always drains.
#include <string.h>

#include <algorithm>
#include <mutex>

#include "score_common.h"

namespace sp {
namespace {

constexpr int kCompute = 6;                       // compute waves per block
constexpr int kControl = 2;                       // control waves (even / odd problems)
constexpr int kThreads = (kCompute + kControl) * 64;
constexpr int kTPW = 3;                           // tiles per compute wave
constexpr int kTilesPerCta = kCompute * kTPW;     // 18
constexpr int kLag = 2;                           // problems between logits and fold
constexpr int kClearLag = 3;                      // slots of x - 3 are free after merging x
constexpr uint64_t kWaitTicks = 200000000ull;     // wall clock runs at 100 MHz: 2 s
constexpr int kQPad = 8;                          // bf16 padding per staged Q row
constexpr int kMaxCtas = 256;                     // blocks per launch (one per CU)

struct StreamTable {
  int32_t B;        // prompts in this launch
  int32_t p0;       // global index of the first one
  int32_t tok_off[SP_MAX_PROMPTS + 1];   // global token offsets of prompts p0 .. p0 + B
  int32_t cta_off[SP_MAX_PROMPTS + 1];   // block prefix within this launch
};

struct StreamWs {
  uint32_t *hdr;    // [0]: tag of a call that timed out; [1]: tag of the latest
                    // call; [2]: blocks of the running launch that have finished
  uint32_t *slot;   // [P][n_cta][32]: bits of each block's partial lse per row
  uint32_t call_tag;
};

template <int D>
struct Smem {
  f32x4 eprev[kLag][kCompute][kTPW][4][64];   // parked e values (16-byte slots per lane)
  __bf16 q[kRows][D + kQPad];                 // staged Q rows of the next problem
  float2 red[2][kCompute][kRows];             // per-wave (m, z) of a problem, by parity
  float lse[2][kRows];                        // staged row lse, by problem parity
  // Hand-offs between the compute waves and the control waves (no block
  // barrier inside the main loop, so neither side waits for the other
  // unless it needs the other's data). Counters are cumulative.
  int q_seq;         // Q of problems < q_seq has been staged (one at a time)
  int q_used;        // compute waves that have read the staged Q
  int stats_cnt;     // compute waves that have written their statistics
  int posted;        // problems this block has posted
  int lse_ready[2];  // lse[s] holds problem lse_ready[s] - 1 (0: nothing yet)
  int lse_used;      // compute waves that have folded with a staged lse
  int ctl_done;      // control waves that have finished
};

__device__ __forceinline__ int lds_get(const int *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_set(int *p, int v) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // data written before the flag
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int lds_inc(int *p) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  return __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void timeout(const StreamWs &ws) {
  __hip_atomic_store(ws.hdr, ws.call_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (bounded) until *p >= v.
__device__ __forceinline__ void lds_wait_ge(const int *p, int v, const StreamWs &ws) {
  if (lds_get(p) >= v) return;
  const uint64_t t0 = wall_clock64();
  while (lds_get(p) < v) {
    if (wall_clock64() - t0 > kWaitTicks) {
      timeout(ws);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int cta_prompt(const StreamTable &t, int c) {
  int lo = 0, hi = t.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t.cta_off[mid] <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Q rows of one problem, one wave: lane -> (row = lane / 2, half of the
// row); 16-byte vectors.
template <int D> struct QRegs { u32x4 v[D / 16]; };

template <int D>
__device__ __forceinline__ void load_q(QRegs<D> &qr, const AttnShape &s, const __bf16 *q, int b,
                                       int prob, int lane) {
  const int row = lane >> 1, h = lane & 1;
  const int l = prob / s.Hkv, g = prob - l * s.Hkv;
  if (row < s.L * s.G) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(q_row_ptr(q, s, b, l, g, row) + h * (D / 2));
#pragma unroll
    for (int i = 0; i < D / 16; ++i) qr.v[i] = src[i];
  } else {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) qr.v[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int D>
__device__ __forceinline__ void store_q(Smem<D> &sm, const QRegs<D> &qr, int lane) {
  const int row = lane >> 1, h = lane & 1;
  u32x4 *dst = reinterpret_cast<u32x4 *>(&sm.q[row][h * (D / 2)]);
#pragma unroll
  for (int i = 0; i < D / 16; ++i) dst[i] = qr.v[i];
}

// Base-2 lse of a set given by its max and its sum of 2^(x - max).
__device__ __forceinline__ float lse_of(float m, float z) {
  return (m == -INFINITY || !(z > 0.f)) ? -INFINITY : m + log2f(z);
}

// Merge every block's partial lse of one problem: lane l takes rows
// 4 (l % 8) .. 4 (l % 8) + 3 of blocks l / 8, l / 8 + 8, ... (in block order),
// then the eight lanes of a row quad merge by an xor tree (each merge is
// symmetric, so every lane ends with identical bits). Lanes 0..7 return the
// row lse of rows 4 l .. 4 l + 3. Empty slots are read again bypassing the L2.
//
// Buffer loads: the resource covers exactly this prompt's slots of the
// problem, so the loads of blocks past its last one return zeros without
// touching memory, and each load's block offset is a scalar operand (no
// per-load address registers).
__device__ f32x4 gather_lse(const StreamWs &ws, int prob, int n_cta, int c_lo, int n_c, int lane) {
  constexpr int kPer = kMaxCtas / 8;
  constexpr int kStride = 8 * kRows * (int)sizeof(float);   // bytes between a lane's blocks
  const uint32_t *base = ws.slot + ((int64_t)prob * n_cta + c_lo) * kRows;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t *>(base), 0, n_c * kRows * (int)sizeof(float), 0x00020000);
  const int c0 = lane >> 3;
  const int voff = c0 * kRows * (int)sizeof(float) + (lane & 7) * 16;
  u32x4 v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, u * kStride, 0);
  const uint64_t t0 = wall_clock64();
  for (;;) {
    bool ok = true;
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      ok &= (c0 + 8 * u >= n_c) | ((v[u][0] != 0u) & (v[u][1] != 0u) & (v[u][2] != 0u) & (v[u][3] != 0u));
    if (__all(ok)) break;
    if (wall_clock64() - t0 > kWaitTicks) { timeout(ws); break; }
    __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");   // the slots change behind the compiler's back: reload
    // Only the quads with an empty slot; cache policy 16: device-coherent
    // (bypasses this die's L2).
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if ((v[u][0] == 0u) | (v[u][1] == 0u) | (v[u][2] == 0u) | (v[u][3] == 0u))
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, u * kStride, 16);
  }
  // Row max first (exact, so the order does not matter), across the lanes
  // of the row quad too; then one exp per partial and a sum tree. Every
  // combination is of two values, so all lanes of a quad end with the same
  // bits (a + b == b + a).
  f32x4 M = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const bool in = c0 + 8 * u < n_c;
#pragma unroll
    for (int e = 0; e < 4; ++e) M[e] = fmaxf(M[e], in ? __uint_as_float(v[u][e]) : -INFINITY);
  }
#pragma unroll
  for (int off = 8; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) M[e] = fmaxf(M[e], __shfl_xor(M[e], off, 64));
  f32x4 Z = {0.f, 0.f, 0.f, 0.f};
  f32x4 Ms;   // M, or 0 where the row has no keys (keeps the exps finite)
#pragma unroll
  for (int e = 0; e < 4; ++e) Ms[e] = M[e] == -INFINITY ? 0.f : M[e];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const bool in = c0 + 8 * u < n_c;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      Z[e] += in ? __builtin_amdgcn_exp2f(__uint_as_float(v[u][e]) - Ms[e]) : 0.f;
  }
#pragma unroll
  for (int off = 8; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) Z[e] += __shfl_xor(Z[e], off, 64);
  f32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = lse_of(M[e], Z[e]);
  return out;
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void k_stream(AttnShape s, StreamTable tb,
                                                        int64_t total_keys, int n_cta,
                                                        const __bf16 *__restrict__ q,
                                                        const __bf16 *__restrict__ k,
                                                        float *__restrict__ imp, StreamWs ws) {
  __shared__ Smem<D> sm;
  const int cta = blockIdx.x;
  // The wave index is uniform across a wave; saying so keeps every value
  // derived from it in scalar registers and every branch on it scalar.
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, r = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool control = wave >= kCompute;
  const int bb = cta_prompt(tb, cta), b = tb.p0 + bb;
  const int c_lo = tb.cta_off[bb], n_c = tb.cta_off[bb + 1] - c_lo, ci = cta - c_lo;
  const int N = tb.tok_off[bb + 1] - tb.tok_off[bb];
  const int NK = N + s.L;                                   // keys of the prompt
  const int tiles = (NK + kTile - 1) / kTile;
  const int ta = (int)((int64_t)tiles * ci / n_c);
  const int nt = (int)((int64_t)tiles * (ci + 1) / n_c) - ta;
  const int64_t key0 = (int64_t)tb.tok_off[bb] + (int64_t)b * s.L;
  const int P = s.n_layers * s.Hkv;

  if (control) {
    // ---------------- control waves: merges, Q staging ----------------
    // Control wave c takes the problems x = c, c + 2, ...: once the compute
    // waves' statistics of x are in, it stages Q(x + 1) (prefetched into its
    // registers), then reads every block's partials of x, merges them and
    // stages the row lse of x. Each control wave thus has two problems'
    // time for one such round.
    const int cw = wave - kCompute;
    QRegs<D> qn;
    if (cw == 0) {
      load_q(qn, s, q, b, 0, lane);
      store_q(sm, qn, lane);
      if (lane == 0) {
        sm.q_used = 0;
        sm.stats_cnt = 0;
        sm.posted = 0;
        sm.lse_ready[0] = 0;
        sm.lse_ready[1] = 0;
        sm.lse_used = 0;
        sm.ctl_done = 0;
        lds_set(&sm.q_seq, 1);
        __hip_atomic_store(ws.hdr + 1, ws.call_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (cw + 1 < P) load_q(qn, s, q, b, cw + 1, lane);
    __syncthreads();
    for (int x = cw; x < P; x += kControl) {
      lds_wait_ge(&sm.stats_cnt, kCompute * (x + 1), ws);
      if (x + 1 < P) {
        lds_wait_ge(&sm.q_used, kCompute * (x + 1), ws);   // Q(x) read by all
        store_q(sm, qn, lane);
        if (lane == 0) lds_set(&sm.q_seq, x + 2);
      }
      lds_wait_ge(&sm.posted, x + 1, ws);                   // our own partial is out
      const f32x4 lq = gather_lse(ws, x, n_cta, c_lo, n_c, lane);
      // The Q prefetch goes out after the gather's loads, so their wait
      // does not include it.
      if (x + 1 + kControl < P) load_q(qn, s, q, b, x + 1 + kControl, lane);
      if (x >= 2) lds_wait_ge(&sm.lse_used, kCompute * (x - 1), ws);   // slot is free
      if (lane < 8) *reinterpret_cast<f32x4 *>(&sm.lse[x & 1][4 * lane]) = lq;
      if (lane == 0) lds_set(&sm.lse_ready[x & 1], x + 1);
      // Every block has read our partials of x - 3: leave them empty.
      if (x >= kClearLag && lane < kRows)
        ws.slot[((int64_t)(x - kClearLag) * n_cta + cta) * kRows + lane] = 0u;
    }
    // The last control wave of the last block out empties the slots of the
    // final problems, which no block can clear earlier.
    const int order = __builtin_amdgcn_readfirstlane(lane == 0 ? lds_inc(&sm.ctl_done) : 0);
    if (order == kControl - 1) {
      const uint32_t done = __builtin_amdgcn_readfirstlane(
          lane == 0 ? __hip_atomic_fetch_add(ws.hdr + 2, 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)
                    : 0u);
      if (done == gridDim.x - 1) {
        const int x0 = P > kClearLag ? P - kClearLag : 0;
        const int n16 = (P - x0) * n_cta * kRows / 4;
        u32x4 *tail = reinterpret_cast<u32x4 *>(ws.slot + (int64_t)x0 * n_cta * kRows);
        for (int i = lane; i < n16; i += 64) tail[i] = u32x4{0u, 0u, 0u, 0u};
        if (lane == 0) __hip_atomic_store(ws.hdr + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  }

  // ---------------- compute waves ----------------
  const int w_t0 = ta + (nt * wave) / kCompute;
  const int w_nt = ta + (nt * (wave + 1)) / kCompute - w_t0;
  const int rows = s.L * s.G;
  const bool row_ok = r < rows;
  const int jr = row_ok ? r / s.G : 0;
  const float sl2 = s.scale_log2;
  // K addressing: a per-problem base pointer plus a 32-bit per-lane element
  // offset of each tile's key row (clamped into the prompt; keys outside the
  // wave's tiles are masked later). Loads are unconditional, which keeps
  // the compiler's wait counts exact: a tile's MFMAs wait for its loads only.
  const int64_t kstride_l = total_keys * s.Hkv * D;   // elements per layer
  uint32_t koff[kTPW];
#pragma unroll
  for (int t = 0; t < kTPW; ++t) {
    const int key = min((w_t0 + t) * kTile + r, NK - 1);
    koff[t] = (uint32_t)((int64_t)key * s.Hkv * D) + 8u * half;
  }
  const __bf16 *kprompt = k + key0 * s.Hkv * D;
  // A tile is "full" when all its keys are prompt keys: no masking needed.
  const int full_tiles = max(0, min((N - w_t0 * kTile) / kTile, w_nt));

  Frag<__bf16, D> kf[kTPW];
  f32x16 E[kTPW], run[kTPW];
#pragma unroll
  for (int t = 0; t < kTPW; ++t) run[t] = f32x16{};
  // Per-tile reference maxima of the problems waiting to be folded:
  // mref[a][t] belongs to problem it - a (a = 0 is the current one).
  float mref[kLag + 1][kTPW];
#pragma unroll
  for (int a = 0; a <= kLag; ++a)
#pragma unroll
    for (int t = 0; t < kTPW; ++t) mref[a][t] = -INFINITY;

  // Ordinary cached loads: one load instruction reads 32 bytes of each of
  // the tile's 32 key rows, so four consecutive instructions share every
  // 128-byte line; a streaming (non-temporal) hint lets the line go between
  // them and costs a refetch each time.
  auto load_k = [&](const __bf16 *kb, int t) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(kb + koff[t]);
#pragma unroll
    for (int st = 0; st < Frag<__bf16, D>::kSteps; ++st)
      kf[t].v[st] = p[2 * st];
  };

#pragma unroll
  for (int t = 0; t < kTPW; ++t) load_k(kprompt, t);
  __syncthreads();

  const u32x4 *qs = reinterpret_cast<const u32x4 *>(&sm.q[r][0]) + half;
  int ln = 0, gn = 0;     // (layer, group) of the next problem to load

  for (int it = 0; it < P + kLag; ++it) {
    const int slot = it % kLag;
#pragma unroll
    for (int a = kLag; a > 0; --a)
#pragma unroll
      for (int t = 0; t < kTPW; ++t) mref[a][t] = mref[a - 1][t];
    if (it < P) {
      // Q of this problem is read from LDS at each k-step of each tile (a
      // register copy would not fit), so the staging buffer is released
      // after the last tile's MFMAs.
      lds_wait_ge(&sm.q_seq, it + 1, ws);
      // Base of the next problem's K (the last problem reloads its own).
      if (it + 1 < P && ++gn == s.Hkv) { gn = 0; ++ln; }
      const __bf16 *kb_next = kprompt + ln * kstride_l + gn * D;
      float m = -INFINITY, z = 0.f;    // base-2 running max and sum of this lane's keys
#pragma unroll
      for (int t = 0; t < kTPW; ++t) {
        asm volatile("" ::: "memory");   // keep the Q reads inside the tile
        f32x16 x = {};
#pragma unroll
        for (int st = 0; st < Frag<__bf16, D>::kSteps; ++st)
          x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[t].v[st]),
                                                     __builtin_bit_cast(bf16x8, qs[2 * st]), x, 0,
                                                     0, 0);
        if (t == kTPW - 1 && lane == 0) lds_inc(&sm.q_used);
        load_k(kb_next, t);
        if (t < full_tiles) {
          // All keys are prompt keys, seen by every row: no masks. (Padding
          // rows compute harmless values that are never folded.)
          float mt = x[0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mt = fmaxf(mt, x[i]);
          const float mn = fmaxf(m, mt * sl2);
          z = m == -INFINITY ? 0.f : z * __builtin_amdgcn_exp2f(m - mn);
          m = mn;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], sl2, -m));
            z += e;
            E[t][i] = e;
          }
        } else {
          // Tail tile: invalid keys, causal lookahead keys, padding rows.
          float mt = -INFINITY;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = (w_t0 + t) * kTile + acc_row(i, half);
            const bool ok = row_ok && t < w_nt && key <= N + jr;   // causal; implies key < NK
            x[i] = ok ? x[i] * sl2 : -INFINITY;
            mt = fmaxf(mt, x[i]);
          }
          const float mn = fmaxf(m, mt);
          if (mn != -INFINITY) {
            z = m == -INFINITY ? 0.f : z * __builtin_amdgcn_exp2f(m - mn);
            m = mn;
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float e = x[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[i] - m);
            z += e;
            const int key = (w_t0 + t) * kTile + acc_row(i, half);
            E[t][i] = key < N ? e : 0.f;    // lookahead keys get no importance
          }
        }
        mref[0][t] = m;
      }
      // Merge the two wave halves (same row, different keys) and hand the
      // wave's statistics to the control wave.
      const float mo = __shfl_xor(m, 32, 64), zo = __shfl_xor(z, 32, 64);
      stats_merge(m, z, mo, zo);
      if (lane < 32) sm.red[it & 1][wave][r] = make_float2(m, z);
      // The last wave to finish the problem posts the block's partials.
      const int arrived = __builtin_amdgcn_readfirstlane(lane == 0 ? lds_inc(&sm.stats_cnt) : 0);
      if (arrived == kCompute * (it + 1) - 1) {
        if (lane < kRows) {
          float M = -INFINITY, Z = 0.f;
#pragma unroll
          for (int w = 0; w < kCompute; ++w)
            stats_merge(M, Z, sm.red[it & 1][w][lane].x, sm.red[it & 1][w][lane].y);
          const uint32_t bits = __float_as_uint(lse_of(M, Z));
          __hip_atomic_store(ws.slot + ((int64_t)it * n_cta + cta) * kRows + lane,
                             bits ? bits : 0x80000000u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane == 0) lds_set(&sm.posted, it + 1);
      }
    }
    if (it >= kLag) {
      // Fold problem it - kLag once its lse is staged: p = e * 2^(m_tile -
      // lse), max into run; then its LDS slot takes this problem's e (same
      // lane, in order).
      lds_wait_ge(&sm.lse_ready[(it - kLag) & 1], it - kLag + 1, ws);
      const float l2 = sm.lse[(it - kLag) & 1][r];
      if (lane == 0) lds_inc(&sm.lse_used);
#pragma unroll
      for (int t = 0; t < kTPW; ++t) {
        const float mr = mref[kLag][t];
        const float f = (row_ok && mr != -INFINITY) ? __builtin_amdgcn_exp2f(mr - l2) : 0.f;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 e = sm.eprev[slot][wave][t][i4][lane];
#pragma unroll
          for (int c = 0; c < 4; ++c) run[t][4 * i4 + c] = fmaxf(run[t][4 * i4 + c], e[c] * f);
        }
      }
    }
    if (it < P) {
#pragma unroll
      for (int t = 0; t < kTPW; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          sm.eprev[slot][wave][t][i4][lane] =
              f32x4{E[t][4 * i4], E[t][4 * i4 + 1], E[t][4 * i4 + 2], E[t][4 * i4 + 3]};
    }
  }

  // Max over the G heads of each step (lanes j*G .. j*G+G-1), then the sum
  // over the steps (the other lane bits; padding rows hold 0): one butterfly
  // over the five lane bits of the row, each level a max or a sum.
#pragma unroll
  for (int lvl = 0; lvl < 5; ++lvl) {
    const int off = 1 << lvl;
    const bool head = off < s.G;
#pragma unroll
    for (int t = 0; t < kTPW; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float o = __shfl_xor(run[t][i], off, 64);
        run[t][i] = head ? fmaxf(run[t][i], o) : run[t][i] + o;
      }
  }
  if (r == 0) {
    float *out = imp + tb.tok_off[bb];
#pragma unroll
    for (int t = 0; t < kTPW; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = (w_t0 + t) * kTile + acc_row(i, half);
        if (t < w_nt && key < N) out[key] = run[t][i] / (float)s.L;
      }
    }
  }
}

struct DeviceInfo {
  int cus = 0;
  int occ64 = 0, occ128 = 0;
};

const DeviceInfo &device_info() {
  static DeviceInfo info[64];
  static bool done[64];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return info[0];
  std::lock_guard<std::mutex> lock(mu);
  if (!done[dev]) {
    DeviceInfo d;
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.occ64, k_stream<64>, kThreads, 0) !=
            hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.occ128, k_stream<128>, kThreads, 0) !=
            hipSuccess)
      d = DeviceInfo();
    info[dev] = d;
    done[dev] = true;
  }
  return info[dev];
}

// Split the batch into launches and give each prompt blocks in proportion to
// its tiles (each block <= 18 tiles). Returns false if a prompt is too long.
struct Plan {
  int n_launch = 0;
  StreamTable t[SP_MAX_PROMPTS];
  int grid[SP_MAX_PROMPTS];
};

bool make_plan(const SegTable &tok, int L, int n_cta, Plan &plan) {
  plan.n_launch = 0;
  int b = 0;
  while (b < tok.B) {
    const int p0 = b;
    int used = 0;
    int need[SP_MAX_PROMPTS];
    int tiles[SP_MAX_PROMPTS];
    while (b < tok.B) {
      const int n = tok.tok_off[b + 1] - tok.tok_off[b];
      const int tl = (n + L + kTile - 1) / kTile;
      const int nd = (tl + kTilesPerCta - 1) / kTilesPerCta;
      if (nd > n_cta) return false;
      if (used + nd > n_cta) break;
      tiles[b - p0] = tl;
      need[b - p0] = nd;
      used += nd;
      ++b;
    }
    const int B = b - p0;
    // Hand out the spare blocks one at a time to the prompt whose blocks
    // carry the most tiles (never more blocks than tiles).
    int spare = n_cta - used;
    while (spare > 0) {
      int best = -1, best_load = 1;
      for (int i = 0; i < B; ++i) {
        if (need[i] >= tiles[i]) continue;
        const int load = (tiles[i] + need[i] - 1) / need[i];
        if (load > best_load) { best = i; best_load = load; }
      }
      if (best < 0) break;
      ++need[best];
      --spare;
    }
    StreamTable &t = plan.t[plan.n_launch];
    memset(&t, 0, sizeof(t));
    t.B = B;
    t.p0 = p0;
    t.cta_off[0] = 0;
    for (int i = 0; i < B; ++i) {
      t.tok_off[i] = tok.tok_off[p0 + i];
      t.cta_off[i + 1] = t.cta_off[i] + need[i];
    }
    t.tok_off[B] = tok.tok_off[p0 + B];
    plan.grid[plan.n_launch] = t.cta_off[B];
    ++plan.n_launch;
  }
  return true;
}

int stream_ctas(const AttnShape &s) {
  const DeviceInfo &d = device_info();
  const int occ = s.d == 128 ? d.occ128 : d.occ64;
  if (occ < 1 || d.cus < 1) return 0;
  return std::min(d.cus, kMaxCtas);
}

}  // namespace

bool score_stream_supported(const AttnShape &s) {
  if (s.dtype != SP_DTYPE_BF16) return false;
  if (s.G & (s.G - 1)) return false;                 // head groups of 2^k lanes
  return true;
}

size_t score_stream_slot_bytes(const AttnShape &s) {
  if (!score_stream_supported(s)) return 0;
  return align_up((size_t)s.n_layers * s.Hkv * kMaxCtas * kRows * sizeof(uint32_t));
}

hipError_t launch_score_stream(const AttnShape &s, const SegTable &tiles, const void *q,
                               const void *k, float *imp, void *ws, hipStream_t st,
                               bool *supported) {
  *supported = false;
  if (!score_stream_supported(s)) return hipSuccess;
  const int n_cta = stream_ctas(s);
  if (n_cta < 1) return hipSuccess;
  static thread_local Plan plan;
  if (!make_plan(tiles, s.L, n_cta, plan)) return hipSuccess;
  *supported = true;
  StreamWs w;
  w.hdr = reinterpret_cast<uint32_t *>(ws);
  w.slot = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(ws) + kStatusBytes);
  w.call_tag = reserve_tags(1);
  const int64_t total_keys = (int64_t)tiles.tok_off[tiles.B] + (int64_t)tiles.B * tiles.L;
  const __bf16 *qp = reinterpret_cast<const __bf16 *>(q);
  const __bf16 *kp = reinterpret_cast<const __bf16 *>(k);
  for (int li = 0; li < plan.n_launch; ++li) {
    if (s.d == 128)
      hipLaunchKernelGGL(k_stream<128>, dim3(plan.grid[li]), dim3(kThreads), 0, st, s, plan.t[li],
                         total_keys, n_cta, qp, kp, imp, w);
    else
      hipLaunchKernelGGL(k_stream<64>, dim3(plan.grid[li]), dim3(kThreads), 0, st, s, plan.t[li],
                         total_keys, n_cta, qp, kp, imp, w);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sp
