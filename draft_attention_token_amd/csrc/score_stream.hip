// Token importance, single-pass streaming form: K is read from HBM once.
//
// Method: "SpecPrefill — Implementation Guide", How It Works / Token
// Importance (max over heads, then layers, then mean over lookahead steps);
// "Speculative prefill" (llama.cpp pull request 27692), Approach steps 2-3.
// Query j of a prompt sits at position N + j and sees keys 0 .. N + j; only
// the N prompt columns receive importance. With the prefill row (the same
// guide's Full Source Code captures the prefill's last row as one more step)
// every step sits one position earlier: step 0 is the prompt's last token and
// sees only the prompt.
//
// Design. A probability needs its row's log-sum-exp (lse) over every key the
// row sees, so no probability is final before all of K has been read. Rather
// than read K twice, the logits stay on chip and the lse arrives later:
//
//  * Persistent grid, one block per CU (a block's shared memory admits only
//    one per unit), all blocks resident at once. Streaming blocks each own
//    <= 18 contiguous 32-key tiles of one prompt for the whole kernel
//    (prompt keys and lookahead keys alike). Eight more blocks, one per chip
//    die (XCD), read no K at all: they do the cross-block merges (below).
//  * The work is a sequence of problems (layer l, KV group g), each with
//    L * G <= 32 query rows (step j, head-in-group hh), padded to 32.
//  * Six compute waves per streaming block, <= 3 tiles each. Per problem a
//    wave computes logits with 32x32x16 bf16 MFMA, K as the A operand (MFMA
//    row = key) and Q as the B operand (MFMA column = query row): a lane
//    holds one query row and 16 keys of each tile, so a row's max and sum
//    over the wave's keys reduce inside the lane plus one swap of wave
//    halves. Statistics are accumulated tile by tile (online max, rescaled
//    sum); each tile's e = 2^(x - m) is relative to the running max m at
//    that tile, kept per tile. A tile's registers are refilled with the next
//    problem's K right after its MFMAs, so the K stream never waits for the
//    cross-block exchange.
//  * The last compute wave to finish a problem merges the six waves'
//    statistics into the block's partial base-2 lse of each row and posts
//    it to the workspace (one float per row).
//  * Exchange, per problem and prompt, in two hops. The prompt's streaming
//    blocks on one die form a group; the merge block of that die waits for
//    the group's partials, merges them and posts the die partial. Every
//    streaming block then merges the (at most eight) die partials itself,
//    in die order, so all get the same bits. The merge blocks issue no K
//    loads, so their reads and posts never queue behind a K stream (a CU
//    serves its vector memory requests roughly in order). Under a full K
//    stream each hop through device-coherent memory costs about two
//    microseconds, which is why there are only two.
//  * Two control waves per streaming block take alternate problems: for
//    problem x a control wave stages Q(x + 1) (prefetched into its
//    registers), then merges the die partials of x and stages the row lse
//    in LDS. Compute and control waves hand data over through LDS flags
//    rather than block barriers, so a late lse only stalls the compute
//    waves when they need it.
//  * The compute waves fold problem i - lag while working on problem i: they
//    park e in LDS (lag problem slots) and turn it into probabilities
//    p = e * 2^(m_tile - lse) once the lse is staged, kept as a running max
//    per (row, key) in registers (max over layers and KV groups). The parked
//    tiles fill the same LDS whatever the lag: 2 problems of 3 tiles per
//    wave, 3 of 2, or 6 of 1. A launch whose blocks own few tiles (shorter
//    prompts) takes the deepest lag that fits, so that more problems pass
//    while the exchange of one is in flight.
//  * Finally: max over the G heads of a step (lanes of a group), mean over
//    the L steps (a butterfly across groups of lanes), store.
//
// Slots. A slot holding all-zero bits has not been posted (a posted value is
// never +0.0: it is stored as -0.0). Slots are left empty for the next
// launch: a streaming block empties its partial of x once it has merged the
// die partials of x (the merge of its group came first), then counts itself
// as a reader of the die partials of (x, prompt); the last reader empties
// them and resets the count. A zero-filled workspace is therefore ready for
// the first launch and stays ready.
//
// Every wait is bounded (about 2 s); on time-out the kernel records it in the
// workspace header and runs to completion, so the grid always drains.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "score_common.h"

namespace sp {
namespace {

constexpr int kCompute = 6;                       // compute waves per block
constexpr int kControl = 2;                       // control waves (even / odd problems)
constexpr int kWaves = kCompute + kControl;
constexpr int kThreads = kWaves * 64;
constexpr int kSlots = 6;                         // parked tiles per wave: lag x tiles per wave
constexpr int kMaxTPW = 3;                        // tiles per compute wave at the shortest lag
constexpr int kTilesPerCta = kCompute * kMaxTPW;  // 18
constexpr uint64_t kWaitTicks = 200000000ull;     // wall clock runs at 100 MHz: 2 s
constexpr int kQPad = 8;                          // bf16 padding per staged Q row
constexpr int kDies = 8;                          // XCDs; block c runs on die c % 8
constexpr int kMaxCtas = 256;                     // blocks per launch (one per CU)
constexpr int kMaxStream = kMaxCtas - kDies;      // streaming blocks per launch
constexpr int kMaxMembers = kMaxStream / kDies;   // streaming blocks per die (31)


struct StreamTable {
  int32_t B;        // prompts in this launch
  int32_t p0;       // global index of the first one
  int32_t n_stream; // streaming blocks 0 .. n_stream - 1
  int32_t merge0;   // merge block of die d: merge0 + d (merge0 % 8 == 0)
  int32_t tok_off[SP_MAX_PROMPTS + 1];   // global token offsets of prompts p0 .. p0 + B
  int32_t cta_off[SP_MAX_PROMPTS + 1];   // streaming-block prefix within this launch
};

// Workspace slots, as uint32 bits of floats (0 = empty). Per problem x:
//   slot, lslot [x][cta][32]          partial lse of each streaming block
//   dslot       [x][prompt][die][32]  die partials
//   readers     [x][prompt]           streaming blocks done with dslot[x][prompt]
struct StreamWs {
  uint32_t *hdr;    // [0]: tag of a call that timed out; [1]: tag of the latest call
  uint32_t *slot;   // device-coherent copy (read by a merge block elsewhere)
  uint32_t *lslot;  // ordinary-store copy (kept in the die's L2)
  uint32_t *dslot;
  uint32_t *readers;
  uint32_t call_tag;
};

__host__ __device__ constexpr int64_t cta_slot(int x, int cta) {
  return ((int64_t)x * kMaxCtas + cta) * kRows;
}
__host__ __device__ constexpr int64_t die_slot(int x, int bb, int die) {
  return (((int64_t)x * SP_MAX_PROMPTS + bb) * kDies + die) * kRows;
}

template <int D, int kLag>
struct Smem {
  f32x4 eprev[kLag][kCompute][kSlots / kLag][4][64];   // parked e (16-byte slots per lane)
  __bf16 q[kRows][D + kQPad];                 // staged Q rows of the next problem
  float2 red[2][kCompute][kRows];             // per-wave (m, z) of a problem, by parity
  float lse[kLag][kRows];                     // staged row lse, by problem mod lag
  // Hand-offs between the compute waves and the control waves (no block
  // barrier inside the main loop, so neither side waits for the other
  // unless it needs the other's data). Counters are cumulative.
  int q_seq;         // Q of problems < q_seq has been staged (one at a time)
  int q_used;        // compute waves that have read the staged Q
  int stats_cnt;     // compute waves that have written their statistics
  int lse_ready[kLag];  // lse[s] holds problem lse_ready[s] - 1 (0: nothing yet)
  int lse_used;      // compute waves that have folded with a staged lse
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
// Device-coherent store (reaches every die).
__device__ __forceinline__ void post(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

template <int D, typename S>
__device__ __forceinline__ void store_q(S &sm, const QRegs<D> &qr, int lane) {
  const int row = lane >> 1, h = lane & 1;
  u32x4 *dst = reinterpret_cast<u32x4 *>(&sm.q[row][h * (D / 2)]);
#pragma unroll
  for (int i = 0; i < D / 16; ++i) dst[i] = qr.v[i];
}

// Base-2 lse of a set given by its max and its sum of 2^(x - max).
__device__ __forceinline__ float lse_of(float m, float z) {
  return (m == -INFINITY || !(z > 0.f)) ? -INFINITY : m + log2f(z);
}

// The streaming blocks of prompt bb on die d: c_lo <= c < c_lo + n_c with
// c % 8 == d, i.e. first, first + 8, ... (size of them, possibly none).
struct Group {
  int first;
  int size;
};

__device__ __forceinline__ Group group_of(int d, int c_lo, int n_c) {
  Group g;
  g.first = c_lo + ((d - c_lo) & (kDies - 1));
  g.size = g.first < c_lo + n_c ? (c_lo + n_c - 1 - g.first) / kDies + 1 : 0;
  return g;
}

// Merge (lse) of up to 4 partials per lane and row, across the lanes of a
// row quad (lane bits 3..5): the max first (exact, order-free), then one exp
// per partial and a sum tree. Every combination is of two values, so all
// lanes of a quad end with the same bits (a + b == b + a).
template <int N>
__device__ __forceinline__ f32x4 merge_quads(const u32x4 (&v)[N], const bool (&in)[N]) {
  f32x4 M = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int u = 0; u < N; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) M[e] = fmaxf(M[e], in[u] ? __uint_as_float(v[u][e]) : -INFINITY);
#pragma unroll
  for (int off = 8; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) M[e] = fmaxf(M[e], __shfl_xor(M[e], off, 64));
  f32x4 Ms;   // M, or 0 where a row has no keys (keeps the exps finite)
#pragma unroll
  for (int e = 0; e < 4; ++e) Ms[e] = M[e] == -INFINITY ? 0.f : M[e];
  f32x4 Z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < N; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      Z[e] += in[u] ? __builtin_amdgcn_exp2f(__uint_as_float(v[u][e]) - Ms[e]) : 0.f;
#pragma unroll
  for (int off = 8; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) Z[e] += __shfl_xor(Z[e], off, 64);
  f32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = lse_of(M[e], Z[e]);
  return out;
}

__device__ __forceinline__ bool quad_full(const u32x4 &v) {
  return (v[0] != 0u) & (v[1] != 0u) & (v[2] != 0u) & (v[3] != 0u);
}

// A slot value is never all-zero bits (the empty mark): +0.0 goes as -0.0.
__device__ __forceinline__ uint32_t slot_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  return u ? u : 0x80000000u;
}

// Loads that see other CUs' stores: cache policy 16 (device scope). Plain
// and policy-1 loads can keep returning a stale line that another CU wrote.
constexpr int kCoherent = 16;

// A merge block's merge of its group's partials of problem x: lane l takes
// rows 4 (l % 8) .. + 3 of members l / 8, l / 8 + 8, ... (member k is block
// first + 8 k, in member order). Polls read the ordinary-store copies, which
// a member on the same die makes visible within about 0.2 us; every eighth
// poll reads the device-coherent copies instead, in case a member runs on
// another die. Buffer loads: the resources cover the group's slots only,
// loads past them return zeros.
__device__ f32x4 gather_group(const StreamWs &ws, int x, const Group &g, int lane) {
  constexpr int kPer = (kMaxMembers + 7) / 8;             // members per lane
  constexpr int kMember = kDies * kRows * (int)sizeof(float);   // bytes between members
  const int64_t at = cta_slot(x, g.first);
  const int bytes = (g.size - 1) * kMember + kRows * (int)sizeof(float);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t *>(ws.lslot + at), 0, bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t *>(ws.slot + at), 0, bytes, 0x00020000);
  const int m0 = lane >> 3;
  const int voff = m0 * kMember + (lane & 7) * 16;
  bool in[kPer];
  u32x4 v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    in[u] = m0 + 8 * u < g.size;
    v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, u * 8 * kMember, kCoherent);
  }
  const uint64_t t0 = wall_clock64();
  for (int round = 1;; ++round) {
    bool ok = true;
#pragma unroll
    for (int u = 0; u < kPer; ++u) ok &= !in[u] | quad_full(v[u]);
    if (__all(ok)) break;
    if (wall_clock64() - t0 > kWaitTicks) { timeout(ws); break; }
    asm volatile("" ::: "memory");   // the slots change behind the compiler's back: reload
    const bool far = (round & 7) == 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (in[u] && !quad_full(v[u]))
        v[u] = far ? __builtin_amdgcn_raw_buffer_load_b128(rg, voff, u * 8 * kMember, kCoherent)
                   : __builtin_amdgcn_raw_buffer_load_b128(rs, voff, u * 8 * kMember, kCoherent);
  }
  return merge_quads(v, in);
}

// A merge block's merge of the die partials of (x, prompt bb): lane l takes
// rows 4 (l % 8) .. + 3 of die l / 8, for the dies set in `dies`.
__device__ f32x4 gather_dies(const StreamWs &ws, int x, int bb, unsigned dies, int lane) {
  const uint32_t *base = ws.dslot + die_slot(x, bb, 0);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t *>(base), 0, kDies * kRows * (int)sizeof(float), 0x00020000);
  const int voff = (lane >> 3) * kRows * (int)sizeof(float) + (lane & 7) * 16;
  const bool in[1] = {((dies >> (lane >> 3)) & 1u) != 0u};
  u32x4 v[1];
  v[0] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, kCoherent);
  const uint64_t t0 = wall_clock64();
  for (;;) {
    if (__all(!in[0] | quad_full(v[0]))) break;
    if (wall_clock64() - t0 > kWaitTicks) { timeout(ws); break; }
    asm volatile("" ::: "memory");
    if (in[0] && !quad_full(v[0]))
      v[0] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, kCoherent);
  }
  return merge_quads(v, in);
}

// Dies holding streaming blocks of a prompt: (c_lo + i) % 8 for i < min(n_c, 8).
__device__ __forceinline__ unsigned prompt_dies(int c_lo, int n_c) {
  if (n_c >= kDies) return 0xffu;
  const unsigned d = ((1u << n_c) - 1u) << (c_lo & (kDies - 1));
  return (d | (d >> kDies)) & 0xffu;
}

// Lanes 0..7 post rows 4 lane .. + 3 of a merged quad (device-coherent).
__device__ __forceinline__ void post_rows(uint32_t *dst, const f32x4 &v, int lane) {
  if (lane < 8) {
#pragma unroll
    for (int e = 0; e < 4; ++e) post(dst + 4 * lane + e, slot_bits(v[e]));
  }
}

// Merge block of die d. Its waves take the (problem, prompt) items x * B + bb
// round robin, in increasing order; an item waits only on smaller ones, so
// every item completes.
__device__ void merge_block(const AttnShape &s, const StreamTable &tb, int d, int wave, int lane,
                            const StreamWs &ws) {
  const int P = s.n_layers * s.Hkv;
  const int items = P * tb.B;
  for (int it = wave; it < items; it += kWaves) {
    const int x = it / tb.B, bb = it - x * tb.B;
    const int c_lo = tb.cta_off[bb], n_c = tb.cta_off[bb + 1] - c_lo;
    const Group g = group_of(d, c_lo, n_c);
    if (g.size == 0) continue;   // the prompt has no blocks on this die
    const f32x4 gl = gather_group(ws, x, g, lane);
    post_rows(ws.dslot + die_slot(x, bb, d), gl, lane);
  }
}

// One level of the final butterfly on every value of the wave's tiles:
// Ctrl >= 0 is a DPP control (within rows of 16 lanes), -1 the swizzle that
// exchanges lane bit 4 (within groups of 32 lanes). Max or sum.
template <int Ctrl, int kTPW>
__device__ __forceinline__ void butterfly_level(f32x16 (&run)[kTPW], bool use_max) {
#pragma unroll
  for (int t = 0; t < kTPW; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int v = __float_as_int(run[t][i]);
      const float o = __int_as_float(Ctrl >= 0 ? __builtin_amdgcn_update_dpp(0, v, Ctrl & 0x1ff, 0xf,
                                                                             0xf, false)
                                               : __builtin_amdgcn_ds_swizzle(v, 0x401f));
      run[t][i] = use_max ? fmaxf(run[t][i], o) : run[t][i] + o;
    }
}

// kF8: K holds fp8 e4m3 codes, key value = kscale[problem] * code; each code
// becomes a bf16 exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1) and the
// scale joins the logit scale of its problem.
template <int D, bool kF8, int kLag>
__global__ __launch_bounds__(kThreads, 1) void k_stream(AttnShape s, StreamTable tb,
                                                        int64_t total_keys,
                                                        const __bf16 *__restrict__ q,
                                                        const uint8_t *__restrict__ k,
                                                        float *__restrict__ imp, StreamWs ws,
                                                        KScales ks) {
  constexpr int kTPW = kSlots / kLag;           // tiles per compute wave
  __shared__ Smem<D, kLag> sm;
  const int cta = blockIdx.x;
  // The wave index is uniform across a wave; saying so keeps every value
  // derived from it in scalar registers and every branch on it scalar.
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, r = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = s.n_layers * s.Hkv;
  if (cta >= tb.n_stream) {
    // Merge blocks, and idle blocks that only pad the merge blocks onto a
    // multiple of 8.
    if (cta >= tb.merge0) merge_block(s, tb, cta - tb.merge0, wave, lane, ws);
    return;
  }
  // The hand-off counters start at zero; the block's only barrier comes
  // before any load, so Q(0) and the first K tiles are fetched together.
  if (tid == 0) {
    sm.q_seq = 0;
    sm.q_used = 0;
    sm.stats_cnt = 0;
    for (int i = 0; i < kLag; ++i) sm.lse_ready[i] = 0;
    sm.lse_used = 0;
    __hip_atomic_store(ws.hdr + 1, ws.call_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const bool control = wave >= kCompute;
  const int bb = cta_prompt(tb, cta), b = tb.p0 + bb;
  const int c_lo = tb.cta_off[bb], n_c = tb.cta_off[bb + 1] - c_lo, ci = cta - c_lo;
  const int N = tb.tok_off[bb + 1] - tb.tok_off[bb];
  const int NK = N + s.La;                                  // keys of the prompt
  // The prompt's keys in tiles of 32 (the last may be partial), dealt to its
  // blocks round-robin: block ci takes tiles ci, ci + n_c, ci + 2 n_c, ...
  // (within one tile of an even share). Every block's stream then spans the
  // whole prompt, which evens out how fast blocks are served (32K keys:
  // 79 -> 72 us against contiguous shares; 128K: 173 -> 170 us).
  const int ntiles = (NK + kTile - 1) / kTile;
  const int nt = (ntiles - ci + n_c - 1) / n_c;
  const int64_t key0 = (int64_t)tb.tok_off[bb] + (int64_t)b * s.La;

  if (control) {
    // ---------------- control waves ----------------
    // Wave kCompute stages Q, wave kCompute + 1 the row lse. Neither waits
    // for the other: a late lse (the cross-block exchange) must not hold up
    // the next problem's Q.
    if (wave == kCompute) {
      // Q(x + 1) goes into the staging buffer once every compute wave has
      // read Q(x) and written its statistics of x (so that no wave starts
      // x + 1 before the last one has counted itself in for x: the last to
      // arrive merges and posts). Two register sets hold the next two
      // problems' Q, loaded two problems ahead (the loads queue behind the
      // block's K stream).
      QRegs<D> qa, qb;
      load_q(qa, s, q, b, 0, lane);
      store_q(sm, qa, lane);
      if (lane == 0) lds_set(&sm.q_seq, 1);
      if (P > 1) load_q(qa, s, q, b, 1, lane);
      if (P > 2) load_q(qb, s, q, b, 2, lane);
      auto stage = [&](int x, QRegs<D> &qr) {   // Q(x + 1), then prefetch Q(x + 3)
        lds_wait_ge(&sm.stats_cnt, kCompute * (x + 1), ws);
        lds_wait_ge(&sm.q_used, kCompute * (x + 1), ws);
        store_q(sm, qr, lane);
        if (lane == 0) lds_set(&sm.q_seq, x + 2);
        if (x + 3 < P) load_q(qr, s, q, b, x + 3, lane);
      };
      for (int x = 0; x + 1 < P; x += 2) {
        stage(x, qa);
        if (x + 2 < P) stage(x + 1, qb);
      }
      return;
    }
    // The lse wave takes the problems in order: merges the die partials of
    // x into the row lse and stages it.
    const unsigned dies = prompt_dies(c_lo, n_c);
    // The last of the prompt's blocks to read the die partials of x empties
    // them (64 lanes x 16 bytes: all eight dies) and the count. A reader
    // learns that it was the last from an atomic whose result it looks at
    // two problems later (it comes back behind the block's K loads).
    uint32_t pend1 = 0u, pend2 = 0u;
    auto last_reader = [&](int x, uint32_t v) {
      if (x < 0 || __builtin_amdgcn_readfirstlane(v) != (uint32_t)n_c - 1u) return;
      uint32_t *dp = ws.dslot + die_slot(x, bb, 0) + 4 * lane;
#pragma unroll
      for (int e = 0; e < 4; ++e) post(dp + e, 0u);
      if (lane == 0) post(ws.readers + (int64_t)x * SP_MAX_PROMPTS + bb, 0u);
    };
    for (int x = 0; x < P; ++x) {
      lds_wait_ge(&sm.stats_cnt, kCompute * (x + 1), ws);   // our own partial of x is out
      last_reader(x - 2, pend2);
      pend2 = pend1;
      const f32x4 lq = gather_dies(ws, x, bb, dies, lane);
      // The slot held lse(x - kLag): free once every compute wave folded it.
      if (x >= kLag) lds_wait_ge(&sm.lse_used, kCompute * (x - kLag + 1), ws);
      if (lane < 8) *reinterpret_cast<f32x4 *>(&sm.lse[x % kLag][4 * lane]) = lq;
      if (lane == 0) lds_set(&sm.lse_ready[x % kLag], x + 1);
      // The merge block of our group has read our partial of x.
      if (lane < kRows) {
        ws.slot[cta_slot(x, cta) + lane] = 0u;
        ws.lslot[cta_slot(x, cta) + lane] = 0u;
      }
      pend1 = lane == 0 ? __hip_atomic_fetch_add(ws.readers + (int64_t)x * SP_MAX_PROMPTS + bb,
                                                 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        : 0u;
    }
    last_reader(P - 2, pend2);
    last_reader(P - 1, pend1);
    return;
  }

  // ---------------- compute waves ----------------
  const int w_t0 = (nt * wave) / kCompute;   // the wave's first tile within the block
  const int w_nt = (nt * (wave + 1)) / kCompute - w_t0;
  // First key of the wave's tile t (t < w_nt): w_key0 + t * t_stride.
  const int t_stride = n_c * kTile;
  const int w_key0 = (ci + n_c * w_t0) * kTile;
  const int rows = s.L * s.G;
  const bool row_ok = r < rows;
  const int jr = row_ok ? r / s.G : 0;
  // K addressing: a per-problem base pointer plus a 32-bit per-lane byte
  // offset of each tile's key row (rows past the prompt's keys read its last
  // key again, tiles past the wave's the wave's first tile, so they cost no
  // traffic, and are masked later). Loads are
  // unconditional, which keeps the compiler's wait counts exact: a tile's
  // MFMAs wait for its loads only.
  // Element layout of the MFMA k-steps (Q in LDS follows the same one):
  //  bf16: step st, half h takes d in [16 st + 8 h, + 8): the lane's loads
  //        are 16 bytes at 32-byte strides;
  //  fp8:  step st, half h takes d in [h D / 2 + 8 st, + 8): the lane reads
  //        its half of the row as D / 32 contiguous 16-byte loads, two steps
  //        per load.
  constexpr int kES = kF8 ? 1 : 2;                  // bytes per K element
  constexpr int kSteps = D / 16;
  constexpr int kLoads = kF8 ? D / 32 : D / 16;     // 16-byte loads per lane and tile
  const int64_t rowb = (int64_t)s.Hkv * D * kES;    // bytes per key row
  const int64_t kstride_l = total_keys * rowb;      // bytes per layer
  uint32_t koff[kTPW];
#pragma unroll
  for (int t = 0; t < kTPW; ++t) {
    const int key = min(w_key0 + (t < w_nt ? t : 0) * t_stride + r, NK - 1);
    koff[t] = (uint32_t)((int64_t)key * rowb) + (uint32_t)(kF8 ? half * (D / 2) : 16 * half);
  }
  const uint8_t *kprompt = k + key0 * rowb;
  // A tile is "full" (no masking needed) when it is one of the wave's and
  // all its keys are prompt keys; the wave's full tiles come first.
  int full_tiles = 0;
  while (full_tiles < w_nt && w_key0 + full_tiles * t_stride + kTile <= N) ++full_tiles;


  u32x4 kf[kTPW][kLoads];
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
  auto load_k = [&](const uint8_t *kb, int t) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(kb + koff[t]);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) kf[t][i] = p[kF8 ? i : 2 * i];
  };
  // The A operand (8 bf16 of the lane's key row) of k-step st of tile t.
  auto k_operand = [&](int t, int st) -> bf16x8 {
    if constexpr (!kF8) {
      return __builtin_bit_cast(bf16x8, kf[t][st]);
    } else {
      const u32x4 w = kf[t][st / 2];
      const uint32_t lo = w[2 * (st % 2)], hi = w[2 * (st % 2) + 1];
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false);
      const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true);
      const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false);
      const bf16x2 d2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true);
      return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d2[0], d2[1]};
    }
  };

#pragma unroll
  for (int t = 0; t < kTPW; ++t) load_k(kprompt, t);

  const u32x4 *qs = reinterpret_cast<const u32x4 *>(&sm.q[r][0]) + (kF8 ? half * (D / 16) : half);
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
      // Base of the next problem's K. After the last problem the loads
      // (unconditional, see above) go to rows that every block of the prompt
      // shares (a lane's row less the block's first tile: the prompt's tiles
      // 0, n_c, 2 n_c, ...), instead of a whole problem again.
      if (it + 1 < P && ++gn == s.Hkv) { gn = 0; ++ln; }
      const uint8_t *kb_next = it + 1 < P ? kprompt + ln * kstride_l + gn * D * kES
                                          : kprompt - (int64_t)ci * kTile * rowb;
      const float sl2 = kF8 ? s.scale_log2 * ks.v[it] : s.scale_log2;
      float m = -INFINITY, z = 0.f;    // base-2 running max and sum of this lane's keys
#pragma unroll
      for (int t = 0; t < kTPW; ++t) {
        asm volatile("" ::: "memory");   // keep the Q reads inside the tile
        f32x16 x = {};
#pragma unroll
        for (int st = 0; st < kSteps; ++st)
          x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              k_operand(t, st), __builtin_bit_cast(bf16x8, qs[kF8 ? st : 2 * st]), x, 0, 0, 0);
        if (t == kTPW - 1 && lane == 0) lds_inc(&sm.q_used);
        // The previous tile's registers take the next problem's K (the
        // wave's last tile after the post): about two thirds of a problem
        // of K in flight per block.
        __builtin_amdgcn_sched_barrier(0);
        if (t > 0) load_k(kb_next, t - 1);
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
            const int key = w_key0 + t * t_stride + acc_row(i, half);
            const bool ok = row_ok && t < w_nt && key < NK && key <= N - s.pre + jr;   // causal
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
            const int key = w_key0 + t * t_stride + acc_row(i, half);
            E[t][i] = (t < w_nt && key < N) ? e : 0.f;    // lookahead keys get no importance
          }
        }
        mref[0][t] = m;
      }
      // Merge the two wave halves (same row, different keys) and hand the
      // wave's statistics over.
      const float mo = __shfl_xor(m, 32, 64), zo = __shfl_xor(z, 32, 64);
      stats_merge(m, z, mo, zo);
      if (lane < 32) sm.red[it & 1][wave][r] = make_float2(m, z);
      // The last wave to finish the problem posts the block's partials.
      const int arrived = __builtin_amdgcn_readfirstlane(lane == 0 ? lds_inc(&sm.stats_cnt) : 0);
      if (arrived == kCompute * (it + 1) - 1 && lane < kRows) {
        float M = -INFINITY, Z = 0.f;
#pragma unroll
        for (int w = 0; w < kCompute; ++w)
          stats_merge(M, Z, sm.red[it & 1][w][lane].x, sm.red[it & 1][w][lane].y);
        // Twice: an ordinary store that the merge block of this die reads
        // from the die's L2, and a device-coherent one for a merge block
        // elsewhere.
        const int64_t at = cta_slot(it, cta) + lane;
        const uint32_t bits = slot_bits(lse_of(M, Z));
        ws.lslot[at] = bits;
        post(ws.slot + at, bits);
      }
      load_k(kb_next, kTPW - 1);
    }
    if (it >= kLag) {
      // Fold problem it - kLag once its lse is staged: p = e * 2^(m_tile -
      // lse), max into run; then its LDS slot takes this problem's e (same
      // lane, in order).
      lds_wait_ge(&sm.lse_ready[(it - kLag) % kLag], it - kLag + 1, ws);
      const float l2 = sm.lse[(it - kLag) % kLag][r];
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
  // over the five lane bits of the row, each level a max or a sum. After
  // level k every aligned group of 2^k lanes holds one value, so a mirror
  // inside the next group pairs the same partial results as an exchange
  // across lane bit k: levels 1, 2 are quad permutations, 4 and 8 the
  // half-row and row mirrors (all DPP), 16 a swizzle within 32 lanes.
  butterfly_level<0xB1>(run, 1 < s.G);
  butterfly_level<0x4E>(run, 2 < s.G);
  butterfly_level<0x141>(run, 4 < s.G);
  butterfly_level<0x140>(run, 8 < s.G);
  butterfly_level<-1>(run, 16 < s.G);
  // Every lane of a half now holds the 16 results of its half's keys; lane
  // r < 16 stores result r, so each tile is one store instruction.
  const float inv_l = 1.f / (float)s.L;
  float *out = imp + tb.tok_off[bb];
#pragma unroll
  for (int t = 0; t < kTPW; ++t) {
    float v = run[t][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) v = r == i ? run[t][i] : v;
    const int key = w_key0 + t * t_stride + acc_row(r & 15, half);
    if (r < 16 && t < w_nt && key < N) out[key] = v * inv_l;
  }
}

struct DeviceInfo {
  int cus = 0;
  int occ64 = 0, occ128 = 0;
  int occ_deep = 0;   // the deepest-lag form (the most shared memory)
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
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.occ64, k_stream<64, false, 2>, kThreads,
                                                     0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.occ128, k_stream<128, false, 2>, kThreads,
                                                     0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.occ_deep, k_stream<128, false, 6>,
                                                     kThreads, 0) != hipSuccess)
      d = DeviceInfo();
    info[dev] = d;
    done[dev] = true;
  }
  return info[dev];
}

// Split the batch into launches and give each prompt streaming blocks in
// proportion to its tiles (each block <= 18 tiles); the merge blocks follow
// at the next multiple of 8. Returns false if a prompt is too long.
struct Plan {
  int n_launch = 0;
  StreamTable t[SP_MAX_PROMPTS];
  int grid[SP_MAX_PROMPTS];
  int max_tiles[SP_MAX_PROMPTS];   // most tiles a streaming block of the launch owns
};

bool make_plan(const SegTable &tok, int L, int n_stream, Plan &plan) {
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
      if (nd > n_stream) return false;
      if (used + nd > n_stream) break;
      tiles[b - p0] = tl;
      need[b - p0] = nd;
      used += nd;
      ++b;
    }
    const int B = b - p0;
    // Hand out the spare blocks one at a time to the prompt whose blocks
    // carry the most tiles (never more blocks than tiles).
    int spare = n_stream - used;
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
    // A block owns ceil(keys / blocks) keys at most, counted in tiles from
    // its first key.
    int most = 1;
    for (int i = 0; i < B; ++i) {
      const int nk = tok.tok_off[p0 + i + 1] - tok.tok_off[p0 + i] + L;
      most = std::max(most, ((nk + need[i] - 1) / need[i] + kTile - 1) / kTile);
    }
    plan.max_tiles[plan.n_launch] = most;
    t.n_stream = t.cta_off[B];
    t.merge0 = (t.n_stream + kDies - 1) / kDies * kDies;
    plan.grid[plan.n_launch] = t.merge0 + kDies;
    ++plan.n_launch;
  }
  return true;
}

// Streaming blocks per launch: the CUs (whole dies' worth) minus the merge
// blocks, so that every block of a launch is resident at once.
int stream_ctas(const AttnShape &s) {
  const DeviceInfo &d = device_info();
  const int occ = std::min(s.d == 128 ? d.occ128 : d.occ64, d.occ_deep);
  if (occ < 1 || d.cus < 2 * kDies) return 0;
  return std::min(d.cus / kDies * kDies, kMaxCtas) - kDies;
}

size_t cta_region(const AttnShape &s) {
  return align_up((size_t)s.n_layers * s.Hkv * kMaxCtas * kRows * sizeof(uint32_t));
}
size_t readers_region(const AttnShape &s) {
  return align_up((size_t)s.n_layers * s.Hkv * SP_MAX_PROMPTS * sizeof(uint32_t));
}
size_t die_region(const AttnShape &s) {
  return align_up((size_t)s.n_layers * s.Hkv * SP_MAX_PROMPTS * kDies * kRows * sizeof(uint32_t));
}

}  // namespace

bool score_stream_supported(const AttnShape &s) {
  if (s.dtype != SP_DTYPE_BF16 && s.dtype != SP_DTYPE_BF16_FP8K) return false;
  if (s.row_pool > 1) return false;                   // pool-before-max: two-pass kernels
  if (s.G & (s.G - 1)) return false;                 // head groups of 2^k lanes
  return true;
}

size_t score_stream_slot_bytes(const AttnShape &s) {
  if (!score_stream_supported(s)) return 0;
  return 2 * cta_region(s) + die_region(s) + readers_region(s);
}

hipError_t launch_score_stream(const AttnShape &s, const SegTable &tiles, const void *q,
                               const void *k, const KScales &ks, float *imp, void *ws,
                               hipStream_t st, bool *supported) {
  *supported = false;
  if (!score_stream_supported(s)) return hipSuccess;
  const int n_stream = stream_ctas(s);
  if (n_stream < 1) return hipSuccess;
  static thread_local Plan plan;
  if (!make_plan(tiles, s.La, n_stream, plan)) return hipSuccess;
  // Lanes address K by 32-bit byte offsets from their prompt's first key row.
  const int64_t rowb = (int64_t)s.Hkv * s.d * (s.dtype == SP_DTYPE_BF16_FP8K ? 1 : 2);
  for (int b = 0; b < tiles.B; ++b) {
    const int64_t nk = (int64_t)tiles.tok_off[b + 1] - tiles.tok_off[b] + s.La;
    if (nk * rowb + rowb > (int64_t)UINT32_MAX) return hipSuccess;
  }
  *supported = true;
  StreamWs w;
  char *base = reinterpret_cast<char *>(ws);
  w.hdr = reinterpret_cast<uint32_t *>(base);
  base += kStatusBytes;
  w.slot = reinterpret_cast<uint32_t *>(base);
  w.lslot = reinterpret_cast<uint32_t *>(base + cta_region(s));
  w.dslot = reinterpret_cast<uint32_t *>(base + 2 * cta_region(s));
  w.readers = reinterpret_cast<uint32_t *>(base + 2 * cta_region(s) + die_region(s));
  w.call_tag = reserve_tags(1);
  const int64_t total_keys = (int64_t)tiles.tok_off[tiles.B] + (int64_t)tiles.B * tiles.L;
  const __bf16 *qp = reinterpret_cast<const __bf16 *>(q);
  const uint8_t *kp = reinterpret_cast<const uint8_t *>(k);
  const bool f8 = s.dtype == SP_DTYPE_BF16_FP8K;
  for (int li = 0; li < plan.n_launch; ++li) {
    // The deepest lag whose tiles per wave cover the launch's largest block.
    const int need_tpw = (plan.max_tiles[li] + kCompute - 1) / kCompute;
    const int lag = need_tpw <= 1 ? 6 : need_tpw == 2 ? 3 : 2;
    auto pick = [&](auto d_tag, auto f8_tag) {
      constexpr int Dv = decltype(d_tag)::value;
      constexpr bool F8v = decltype(f8_tag)::value;
      return lag == 6 ? k_stream<Dv, F8v, 6> : lag == 3 ? k_stream<Dv, F8v, 3> : k_stream<Dv, F8v, 2>;
    };
    using D64 = std::integral_constant<int, 64>;
    using D128 = std::integral_constant<int, 128>;
    auto kern = s.d == 128 ? (f8 ? pick(D128{}, std::true_type{}) : pick(D128{}, std::false_type{}))
                           : (f8 ? pick(D64{}, std::true_type{}) : pick(D64{}, std::false_type{}));
    hipLaunchKernelGGL(kern, dim3(plan.grid[li]), dim3(kThreads), 0, st, s, plan.t[li], total_keys,
                       qp, kp, imp, w, ks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sp
