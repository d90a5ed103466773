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
// than read K twice, each block keeps the exponentiated logits of its keys on
// chip until the row lse arrives from the other blocks:
//
//  * Persistent grid, one block per CU, all blocks resident at once (the
//    host checks that the grid fits). Streaming blocks share a prompt's 32-key tiles
//    round-robin (block i of n takes tiles i, i + n, ...), at most 21 each.
//    Eight more blocks, one per chip die (XCD), read no K: they merge the
//    partial results of the streaming blocks on their die.
//  * The work is a sequence of problems (layer l, KV group g), each with
//    S * G <= 32 query rows (step j, head-in-group hh), padded to 32.
//  * Seven compute waves per streaming block, <= 3 tiles each, and one
//    control wave. K reaches LDS by direct loads (global -> LDS, no
//    registers): every load instruction reads whole 128-byte lines, eight
//    lanes per line, with the non-temporal hint. Each compute wave streams
//    its own tiles through a ring of four 4 KB units (32 keys x 128 bytes),
//    refilling a unit as soon as its MFMAs have read it. The chunks of a key
//    are stored XOR-swizzled, so the MFMA operand reads (16 bytes of 32 key
//    rows) hit distinct LDS banks.
//  * Per problem a compute wave computes logits with 32x32x16 bf16 MFMA, K as
//    the A operand (row = key) and Q as the B operand (column = query row;
//    with bf16 K its operands are read from LDS with each unit's K operands,
//    with fp8 K into registers at the start of the problem): a lane
//    holds one query row and 16 keys of each tile, 16 fp32 accumulators per
//    tile. After the MFMAs the wave takes each row's max over its keys,
//    turns the logits in place into e = 2^(x - m) and sums them, then parks
//    e in 24-bit form (the rounded float's top three bytes) until the row
//    lse is known. A wave keeps kPk problems parked, the most its registers
//    hold: 3 at 3 tiles per wave (2 with small groups), 4 at 2
//    tiles, 7 at 1.
//  * The last compute wave to finish a problem merges the seven waves'
//    statistics into the block's partial base-2 lse of each row and posts it
//    to the workspace.
//  * Exchange, per problem and prompt, in two hops. The prompt's streaming
//    blocks on one die form a group; the merge block of that die waits for
//    the group's partials, merges them and posts the die partial. The
//    control wave of every streaming block merges the (at most eight) die
//    partials, in die order, so all blocks get the same bits, and stages the
//    row lse in LDS. It also stages each problem's Q in LDS, three problems
//    ahead. Its own load queue holds only these, so its polls never wait
//    behind the K stream.
//  * Before parking problem x in its slot, the wave folds the slot's
//    previous occupant, problem x - kPk: p = e * 2^(m - lse), the max over
//    the heads on the lane bits that hold them, and the max into a running
//    value per (row, key) in registers (the max over layers and KV groups).
//  * Finally: the rest of the max over the G heads of a step, the mean over
//    the steps (a butterfly across groups of lanes), store.
//
// Slots carry the tag of the call that posted them, next to the value, so a
// waiting block only takes values of its own call: nothing needs clearing
// between calls, and a call that gave up leaves nothing that a later call
// could mistake for its own. Every wait is bounded (2 s unless the host sets
// another budget); on time-out the kernel records it in the workspace header
// and runs to completion, so the grid always drains.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "score_common.h"

namespace sp {
namespace {

constexpr int kCompute = 7;                       // compute waves per streaming block
constexpr int kWaves = kCompute + 1;              // + the control wave
constexpr int kThreads = kWaves * 64;
constexpr int kRing = 4;                          // K units in each compute wave's ring
constexpr int kUnitBytes = 4096;                  // 32 keys x 128 bytes
constexpr int kQSlots = 3;                        // staged Q problems
constexpr int kQSlotBytes = 8192;                 // 32 rows x 128 bf16
constexpr int kLseSlots = 8;                      // staged row lse (>= the deepest lag)
constexpr int kRedSlots = 4;                      // per-wave statistics of problems in flight
constexpr int kMaxTPW = 3;                        // tiles per compute wave
constexpr int kTilesPerCta = kCompute * kMaxTPW;  // 21
constexpr int kDies = 8;                          // XCDs; block c runs on die c % 8
constexpr int kMaxCtas = 256;                     // blocks per launch (one per CU)
constexpr int kMaxStream = kMaxCtas - kDies;      // streaming blocks per launch
constexpr int kMaxMembers = kMaxStream / kDies;   // streaming blocks per die (31)
constexpr uint32_t kOob = 0xFFFFFFF0u;            // a buffer offset past every resource

struct StreamTable {
  int32_t B;        // prompts in this launch
  int32_t p0;       // global index of the first one
  int32_t n_stream; // streaming blocks 0 .. n_stream - 1
  int32_t merge0;   // merge block of die d: merge0 + d (merge0 % 8 == 0)
  int32_t tok_off[SP_MAX_PROMPTS + 1];   // global token offsets of prompts p0 .. p0 + B
  int32_t cta_off[SP_MAX_PROMPTS + 1];   // streaming-block prefix within this launch
};

// Workspace slots: 64-bit words, the low half a float's bits, the high half
// the tag of the call that wrote it. Per problem x:
//   slot, lslot [x][cta][32]          partial lse of each streaming block
//   dslot       [x][prompt][die][32]  die partials
struct StreamWs {
  uint32_t *hdr;    // [0]: tag of a call that timed out; [1]: tag of the latest call
  uint64_t *slot;   // device-coherent copy (read by a merge block elsewhere)
  uint64_t *lslot;  // ordinary-store copy (kept in the die's L2)
  uint64_t *dslot;
  uint32_t call_tag;
  uint64_t wait_ticks;   // budget of each cross-block wait (wall clock, 100 MHz)
};

__host__ __device__ constexpr int64_t cta_slot(int x, int cta) {
  return ((int64_t)x * kMaxCtas + cta) * kRows;
}
__host__ __device__ constexpr int64_t die_slot(int x, int bb, int die) {
  return (((int64_t)x * SP_MAX_PROMPTS + bb) * kDies + die) * kRows;
}

// Shared memory: the K ring and the Q slots (written by direct loads) and
// the control block are separate objects. Loads into shared memory are
// counted as outstanding vector-memory operations; the compiler makes an
// access wait for all of them unless it can tell the access cannot touch
// their destination, which it can only across distinct objects. The ring and
// Q reads wait for exactly their own loads by explicit counts.
struct Ring {
  alignas(16) uint8_t unit[kCompute][kRing][kUnitBytes];   // K units, by wave
};
struct QSlots {
  alignas(16) uint8_t q[kQSlots][kQSlotBytes];             // Q of three problems
};
struct Smem {
  float2 red[kRedSlots][kCompute][kRows];                  // per-wave (m, z), by problem % 4
  float lse[kLseSlots][kRows];                             // staged row lse, by problem % 8
  // Hand-offs between the compute waves and the control wave, without a
  // block barrier inside the main loop. Compute waves may drift apart by up
  // to three problems (a wave needs Q(x + 3), whose slot frees only when
  // every wave has read Q(x): its last MFMA of x with bf16 K), so each
  // counter belongs to a slot and counts
  // the slot's uses cumulatively: 7 per problem that used it.
  int q_ready;                 // Q of problems < q_ready is staged
  int q_used[kQSlots];         // reads of Q slot x % 3 completed
  int stats_cnt[kRedSlots];    // statistics of problems x % 4 written
  int lse_ready[kLseSlots];    // lse[s] holds problem lse_ready[s] - 1 (0: nothing yet)
  int lse_used[kLseSlots];     // folds with lse slot x % 8 done
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
// A wait that gives up records the call's tag in the header; the wave then
// stops waiting altogether (`dead`), so a failed call drains quickly.
__device__ __forceinline__ void timeout(const StreamWs &ws, bool &dead) {
  __hip_atomic_store(ws.hdr, ws.call_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  dead = true;
}

// Wait (bounded) until *p >= v.
__device__ __forceinline__ void lds_wait_ge(const int *p, int v, const StreamWs &ws, bool &dead) {
  if (dead || lds_get(p) >= v) return;
  const uint64_t t0 = wall_clock64();
  while (lds_get(p) < v) {
    if (wall_clock64() - t0 > ws.wait_ticks) {
      timeout(ws, dead);
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

// stats_merge without branches, on the hardware exp2 (terms below 2^-126 of
// the total flush to 0): for the partials of one block.
__device__ __forceinline__ void stats_merge_lean(float &M, float &Z, float m, float z) {
  const float nm = fmaxf(M, m);
  const float a = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - nm);
  const float b = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - nm);
  Z = Z * a + z * b;
  M = nm;
}

// Base-2 lse of a set given by its max and its sum of 2^(x - max).
__device__ __forceinline__ float lse_of(float m, float z) {
  return (m == -INFINITY || !(z > 0.f)) ? -INFINITY : m + log2f(z);
}

// A posted slot: the value's bits and the call's tag.
__device__ __forceinline__ uint64_t slot_word(float v, uint32_t tag) {
  return ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
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

// Kernel forms: the lag (problems folded behind) and the tiles per compute
// wave it allows, 6 to 8 e slots of 16 registers each.
// Problems a compute wave keeps parked (kPk) for the tiles it owns, and
// back: the most that fit its registers. At three tiles that is three,
// except where the running maxima take more registers (CL < 2: two). The fp8
// form with three spills 8 VGPRs and still beats two (the lse of a problem
// arrives about two problems after its statistics: at 128K tokens 112 ->
// 106 us), so it keeps three as well.
__host__ __device__ constexpr int tpw_for_pk(int pk) { return pk <= 3 ? 3 : pk == 4 ? 2 : 1; }
constexpr int pk_for_tpw(int tpw, int cl) { return tpw <= 1 ? 7 : tpw == 2 ? 4 : cl == 2 ? 3 : 2; }

// A lane's four rows of a partial: two 16-byte loads of two slots each.
struct Quad {
  u32x4 a, b;   // {bits, tag, bits, tag} of rows 4q, 4q + 1 and 4q + 2, 4q + 3
};
__device__ __forceinline__ bool quad_full(const Quad &v, uint32_t tag) {
  return (v.a[1] == tag) & (v.a[3] == tag) & (v.b[1] == tag) & (v.b[3] == tag);
}
__device__ __forceinline__ f32x4 quad_values(const Quad &v) {
  return f32x4{__uint_as_float(v.a[0]), __uint_as_float(v.a[2]), __uint_as_float(v.b[0]),
               __uint_as_float(v.b[2])};
}

// Merge (lse) of up to N partials per lane and row, across the lanes of a
// row quad (lane bits 3..5): the max first (exact, order-free), then one exp
// per partial and a sum tree. Every combination is of two values, so all
// lanes of a quad end with the same bits (a + b == b + a).
template <int N>
__device__ __forceinline__ f32x4 merge_quads(const Quad (&v)[N], const bool (&in)[N]) {
  f32x4 M = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const f32x4 x = quad_values(v[u]);
#pragma unroll
    for (int e = 0; e < 4; ++e) M[e] = fmaxf(M[e], in[u] ? x[e] : -INFINITY);
  }
#pragma unroll
  for (int off = 8; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) M[e] = fmaxf(M[e], __shfl_xor(M[e], off, 64));
  f32x4 Ms;   // M, or 0 where a row has no keys (keeps the exps finite)
#pragma unroll
  for (int e = 0; e < 4; ++e) Ms[e] = M[e] == -INFINITY ? 0.f : M[e];
  f32x4 Z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const f32x4 x = quad_values(v[u]);
#pragma unroll
    for (int e = 0; e < 4; ++e) Z[e] += in[u] ? __builtin_amdgcn_exp2f(x[e] - Ms[e]) : 0.f;
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

// Loads that see other CUs' stores: cache policy 16 (device scope). Plain
// and policy-1 loads can keep returning a stale line that another CU wrote.
constexpr int kCoherent = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
// The same from wave-uniform values, placed in scalar registers (an inline
// assembly operand that must live there).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_uniform(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return rsrc(reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo),
              __builtin_amdgcn_readfirstlane(bytes));
}

__device__ __forceinline__ Quad load_quad(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
  Quad q;
  q.a = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kCoherent);
  q.b = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, soff, kCoherent);
  return q;
}

// A merge block's merge of its group's partials of problem x: lane l takes
// rows 4 (l % 8) .. + 3 of members l / 8, l / 8 + 8, ... (member k is block
// first + 8 k, in member order). Polls read the ordinary-store copies, which
// a member on the same die makes visible within about 0.2 us; every eighth
// poll reads the device-coherent copies instead, in case a member runs on
// another die. Buffer loads: the resources cover the group's slots only.
__device__ f32x4 gather_group(const StreamWs &ws, int x, const Group &g, int lane, bool &dead) {
  constexpr int kPer = (kMaxMembers + 7) / 8;                   // members per lane
  constexpr int kMember = kDies * kRows * (int)sizeof(uint64_t);   // bytes between members
  const int64_t at = cta_slot(x, g.first);
  const uint32_t bytes = (g.size - 1) * kMember + kRows * (int)sizeof(uint64_t);
  const __amdgpu_buffer_rsrc_t rs = rsrc(ws.lslot + at, bytes);
  const __amdgpu_buffer_rsrc_t rg = rsrc(ws.slot + at, bytes);
  const int m0 = lane >> 3;
  const uint32_t voff = m0 * kMember + (lane & 7) * 32;
  bool in[kPer];
  Quad v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    in[u] = m0 + 8 * u < g.size;
    v[u] = load_quad(rs, voff, u * 8 * kMember);
  }
  const uint64_t t0 = wall_clock64();
  for (int round = 1;; ++round) {
    bool ok = true;
#pragma unroll
    for (int u = 0; u < kPer; ++u) ok &= !in[u] | quad_full(v[u], ws.call_tag);
    if (__all(ok) || dead) break;
    if (wall_clock64() - t0 > ws.wait_ticks) { timeout(ws, dead); break; }
    asm volatile("" ::: "memory");   // the slots change behind the compiler's back: reload
    const bool far = (round & 7) == 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (in[u] && !quad_full(v[u], ws.call_tag))
        v[u] = load_quad(far ? rg : rs, voff, u * 8 * kMember);
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
__device__ __forceinline__ void post_rows(uint64_t *dst, const f32x4 &v, uint32_t tag, int lane) {
  if (lane < 8) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      __hip_atomic_store(dst + 4 * lane + e, slot_word(v[e], tag), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Merge block of die d. Its waves take the (problem, prompt) items x * B + bb
// round robin, in increasing order; an item waits only on smaller ones, so
// every item completes.
__device__ void merge_block(const AttnShape &s, const StreamTable &tb, int d, int wave, int lane,
                            const StreamWs &ws) {
  const int P = s.n_layers * s.Hkv;
  const int items = P * tb.B;
  bool dead = false;
  for (int it = wave; it < items; it += kWaves) {
    const int x = it / tb.B, bb = it - x * tb.B;
    const int c_lo = tb.cta_off[bb], n_c = tb.cta_off[bb + 1] - c_lo;
    const Group g = group_of(d, c_lo, n_c);
    if (g.size == 0) continue;   // the prompt has no blocks on this die
    const f32x4 gl = gather_group(ws, x, g, lane, dead);
    post_rows(ws.dslot + die_slot(x, bb, d), gl, ws.call_tag, lane);
  }
}

// LDS layout of a unit (32 rows x UB bytes, UB = 128 or 64): one 1 KB block
// per load instruction holding KPI = 1024 / UB consecutive rows; row r's
// 16-byte chunk c sits at chunk position c ^ swz(r) inside the row. With
// SPK = UB / 16 chunks per row, 16 / SPK rows share a 256-byte bank line,
// and the swizzle makes the 16 rows an MFMA operand read touches (one chunk
// each) fall on 16 distinct 16-byte bank groups.
template <int UB>
struct UnitLayout {
  static constexpr int SPK = UB / 16;
  static constexpr int KPI = 1024 / UB;
  static constexpr int IPU = 32 / KPI;   // load instructions per unit
  __device__ static constexpr int swz(int r) { return (r / (16 / SPK)) % SPK; }
  __device__ static constexpr int row_base(int r) { return 1024 * (r / KPI) + UB * (r % KPI); }
};

// Per-call constants a compute wave needs.
struct WaveCtx {
  AttnShape s;
  StreamWs ws;
  const KScales *ks;
  const uint8_t *k;
  float *imp;
  int64_t total_keys, key0;
  int P, N, NK, rows, cta, tok0;
  int w_key0, t_stride, full_tiles;   // the wave's tiles: keys w_key0 + t * t_stride ..
  int wave, lane;
};

// A compute wave that owns NT tiles (0 <= NT <= 3): the tile count is a
// compile-time constant, so every e slot stays in fixed registers with no
// branch around it.
template <int D, bool kF8, int kPk, int CL, int NT>
__device__ __forceinline__ void compute_wave(const WaveCtx &c, Ring &ring, QSlots &qsl, Smem &sm,
                                             bool &dead) {
  constexpr int kES = kF8 ? 1 : 2;                   // bytes per K element
  constexpr int RBG = D * kES;                       // K bytes per key and KV group
  constexpr int UB = RBG < 128 ? RBG : 128;          // bytes per key in a unit
  constexpr int UPT = RBG / UB;                      // units per tile
  constexpr int kSteps = D / 16;                     // MFMA k-steps per tile
  constexpr int kStepsPerUnit = kSteps / UPT;
  using KL = UnitLayout<UB>;
  using QL = UnitLayout<128>;
  constexpr int NTA = NT > 0 ? NT : 1;               // array extent
  const AttnShape &s = c.s;
  const StreamWs &ws = c.ws;
  const int lane = c.lane, half = lane >> 5, r = lane & 31, wave = c.wave;
  const int P = c.P, N = c.N, NK = c.NK;
  const int w_key0 = c.w_key0, t_stride = c.t_stride;
  // Query row r of the group: head r / (32 / G), step r % (32 / G) (heads
  // on the top lane bits, so the head max can start at fold time: below).
  const int rs_h = 32 / s.G;
  const int jr = r % rs_h;
  const bool row_ok = jr < s.L;

  // K of the prompt, by problem: a resource per (layer, group) whose range
  // ends at the prompt's last key row; keys past it read as zeros.
  const int64_t rowb = (int64_t)s.Hkv * RBG;          // bytes per key row (all groups)
  const uint32_t k_bytes = (uint32_t)((NK - 1) * rowb + RBG);
  const int64_t layer_step = c.total_keys * rowb - (int64_t)(s.Hkv - 1) * RBG;
  // Per load instruction i of a unit: the lane's row (key within the tile)
  // and byte offset of its 16-byte chunk.
  const int lrow0 = lane / KL::SPK;            // + KPI i for instruction i
  uint32_t loff[KL::IPU];
#pragma unroll
  for (int i = 0; i < KL::IPU; ++i) {
    const int rr = KL::KPI * i + lrow0;
    loff[i] = (uint32_t)(rr * rowb + 16 * ((lane % KL::SPK) ^ KL::swz(rr)));
  }
  // The ring: unit k of the wave's sequence (problem, tile, unit of the tile)
  // goes to slot k % 4. Issue state, advanced without divisions.
  const int total_units = P * NT * UPT;
  const uint32_t tile_bytes = (uint32_t)(t_stride * rowb);   // between the wave's tiles
  const uint32_t toff0 = (uint32_t)(w_key0 * rowb);
  int ki = 0, kt = 0, ku = 0, kg = 0;            // next unit to issue: its tile, unit, group
  const uint8_t *kbase = c.k + c.key0 * rowb;    // group slice of its problem
  uint32_t ktoff = toff0;                        // its tile's offset
  auto issue_next = [&]() {
    if (ki >= total_units) return;
    const __amdgpu_buffer_rsrc_t kr = rsrc_uniform(kbase, k_bytes);
    const uint32_t tb_off = ktoff + ku * UB;
    const int tk0 = w_key0 + kt * t_stride;    // the tile's first key
    // The loads are issued by inline assembly: the compiler then does not
    // track them, so it adds no waits for them before unrelated shared
    // memory accesses (it would otherwise wait for every outstanding K load
    // before each hand-off counter). wait_unit() waits for them explicitly.
    const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
        (__attribute__((address_space(3))) uint8_t *)&ring.unit[wave][ki & (kRing - 1)][0]));
    if (tk0 + kTile <= NK) {
#pragma unroll
      for (int i = 0; i < KL::IPU; ++i)
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds"
                     :: "v"(tb_off + loff[i]), "s"(kr), "{m0}"(dst + 1024 * i) : "memory");
    } else {
#pragma unroll
      for (int i = 0; i < KL::IPU; ++i) {
        const uint32_t vo = tk0 + KL::KPI * i + lrow0 < NK ? tb_off + loff[i] : kOob;
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds"
                     :: "v"(vo), "s"(kr), "{m0}"(dst + 1024 * i) : "memory");
      }
    }
    ++ki;
    if (++ku == UPT) {
      ku = 0;
      ktoff += tile_bytes;
      if (++kt == NT) {
        kt = 0;
        ktoff = toff0;
        if (++kg == s.Hkv) { kg = 0; kbase += layer_step; } else { kbase += RBG; }
      }
    }
  };
#pragma unroll
  for (int i = 0; i < kRing; ++i) issue_next();
  int kc = 0;   // next unit to consume
  // Wait until unit kc has landed: the (three) units issued after it may
  // still fly; near the end of the stream wait for everything.
  auto wait_unit = [&]() {
    if (ki - kc >= kRing) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kRing - 1) * KL::IPU) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // Operand reads. K: k-step st reads chunk 2 st + half of the row (bf16;
  // unit st / 4) or 8 bytes at half of chunk st (fp8). Q: chunk 2 st + half
  // (unit st / 4). For 128-byte units the two layouts coincide.
  const int k_rb = KL::row_base(r), k_sw = KL::swz(r);
  const int q_rb = QL::row_base(r), q_sw = QL::swz(r);
  auto k_operand = [&](const uint8_t *unit, int st) -> bf16x8 {
    if constexpr (!kF8) {
      const int cc = (2 * st + half) % KL::SPK;
      return *reinterpret_cast<const bf16x8 *>(unit + k_rb + 16 * (cc ^ k_sw));
    } else {
      const int cc = st % KL::SPK;
      const uint2 w = *reinterpret_cast<const uint2 *>(unit + k_rb + 16 * (cc ^ k_sw) + 8 * half);
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, false);
      const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, true);
      const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, false);
      const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, true);
      return bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
    }
  };
  auto q_operand = [&](const uint8_t *qs, int st) -> bf16x8 {
    const int kq = 2 * st + half;
    return *reinterpret_cast<const bf16x8 *>(qs + (kq / 8) * kUnitBytes + q_rb +
                                             16 * ((kq % 8) ^ q_sw));
  };
  // MFMAs of unit u of a tile into acc: the unit's K operands are all read
  // first (one wait for shared memory per unit); Q comes from registers. The
  // unit 0 MFMAs start from init: 0, or -inf where a key is past the
  // prompt's keys or hidden from the row (causality), so the logit is -inf
  // there.
  // Q's operands: with bf16 K they are read from LDS with each unit's K
  // operands and live only during its MFMAs, which leaves more registers to
  // the parked problems (measured faster: 16 prompts 611 -> 604 us, 128K
  // 141.6 -> 141.1 us); fp8 K, which widens its operands in registers, keeps
  // them in registers for the problem (that way 108.1 us against 110.1).
  constexpr bool kQRegs = kF8;
  auto mfma_unit = [&](f32x16 &acc, const uint8_t *unit, const bf16x8 *qreg, const uint8_t *qs,
                       int u, const f32x16 &init) {
    bf16x8 ko[kStepsPerUnit], qo[kQRegs ? 1 : kStepsPerUnit];
#pragma unroll
    for (int j = 0; j < kStepsPerUnit; ++j) {
      ko[j] = k_operand(unit, u * kStepsPerUnit + j);
      if constexpr (!kQRegs) qo[j] = q_operand(qs, u * kStepsPerUnit + j);
    }
#pragma unroll
    for (int j = 0; j < kStepsPerUnit; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ko[j], kQRegs ? qreg[u * kStepsPerUnit + j] : qo[j],
                                                    (u == 0 && j == 0) ? init : acc, 0, 0, 0);
  };
  // Accumulator start of tile t: all 0 unless the tile reaches past the
  // prompt's keys (lookahead keys and the rest of the prompt's last tile).
  // The lane's 16 visible keys of each tile as a bit mask, expanded at use
  // (an opaque step keeps the compiler from hoisting 16 registers per tile
  // out of the problem loop).
  uint32_t vis[NTA];
  bool partial[NTA];
#pragma unroll
  for (int t = 0; t < NTA; ++t) {
    const int tk0 = w_key0 + t * t_stride;
    partial[t] = tk0 + kTile > N;
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = tk0 + acc_row(i, half);
      m |= (key < NK && key <= N - s.pre + jr) ? 1u << i : 0u;
    }
    vis[t] = m;
  }
  auto tile_init = [&](int t) -> f32x16 {
    f32x16 v = {};
    if (partial[t]) {
      uint32_t m = vis[t];
      asm volatile("" : "+v"(m));
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = (m >> i) & 1u ? 0.f : -INFINITY;
    }
    return v;
  };

  // The problem in flight accumulates its logits in ec (16 floats per lane
  // and tile), which the statistics turn into e = 2^(x - m) <= 1. Then e is
  // parked until the row lse of the problem is known, in 24-bit form: the
  // top three bytes of the float after rounding to nearest (15 mantissa
  // bits, relative error <= 2^-16), in slot x % kPk. At the end of problem x
  // the wave folds the slot's previous occupant, problem x - kPk: p =
  // e * 2^(m - lse), max into run, a running max per (row, key) kept as the
  // bits of non-negative floats (they order like the values). The fold also
  // takes the max over the heads on lane bits 4 (and 3): CL levels, after
  // which a lane keeps 16 >> CL of its 16 keys (acc index 8 b4 + 4 b3 + k).
  constexpr int RV = 16 >> CL;
  f32x16 ec[NTA];
  uint32_t pk[kPk][NTA][12];
  float mref[kPk];           // row max of the problem in each slot (base 2)
  uint32_t run[NTA][RV];
#pragma unroll
  for (int t = 0; t < NTA; ++t) {
#pragma unroll
    for (int k = 0; k < RV; ++k) run[t][k] = 0u;
#pragma unroll
    for (int a = 0; a < kPk; ++a)
#pragma unroll
      for (int i = 0; i < 12; ++i) pk[a][t][i] = 0u;
  }
#pragma unroll
  for (int a = 0; a < kPk; ++a) mref[a] = -INFINITY;
  const bool b3 = (lane >> 3) & 1;
  // Four floats (a, b, c, d) -> three words [a1 a2 a3 b1] [b2 b3 c1 c2]
  // [c3 d1 d2 d3] (byte 0 of each float dropped after rounding), and back.
  auto park = [&](const f32x16 &v, uint32_t (&o)[12]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t w0 = __float_as_uint(v[4 * g]) + 0x80u;
      const uint32_t w1 = __float_as_uint(v[4 * g + 1]) + 0x80u;
      const uint32_t w2 = __float_as_uint(v[4 * g + 2]) + 0x80u;
      const uint32_t w3 = __float_as_uint(v[4 * g + 3]) + 0x80u;
      o[3 * g] = __builtin_amdgcn_perm(w1, w0, 0x05030201u);
      o[3 * g + 1] = __builtin_amdgcn_perm(w2, w1, 0x06050302u);
      o[3 * g + 2] = __builtin_amdgcn_perm(w3, w2, 0x07060503u);
    }
  };
  auto unpark = [&](const uint32_t (&o)[12], int i) -> float {
    const int g = i / 4, j = i % 4;
    uint32_t w;
    if (j == 0) w = __builtin_amdgcn_perm(0u, o[3 * g], 0x0201000Cu);
    else if (j == 1) w = __builtin_amdgcn_perm(o[3 * g + 1], o[3 * g], 0x0504030Cu);
    else if (j == 2) w = __builtin_amdgcn_perm(o[3 * g + 2], o[3 * g + 1], 0x0403020Cu);
    else w = __builtin_amdgcn_perm(0u, o[3 * g + 2], 0x0302010Cu);
    return __uint_as_float(w);
  };
  // Fold tile t of slot a into run with factor f (0 for an empty slot: a
  // no-op, since run >= 0).
  auto fold_tile = [&](int a, int t, float f) {
    uint32_t p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __float_as_uint(unpark(pk[a][t], i) * f);
    if constexpr (CL >= 1) {
      // Lane bit 4 (lanes l, l ^ 16): one swap of register pairs (i, i + 8)
      // gives the lane with bit 4 clear both values of key i, the other
      // both values of key i + 8.
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const auto sw = __builtin_amdgcn_permlane16_swap(p[i], p[i + 8], false, false);
        p[i] = __builtin_elementwise_max(sw[0], sw[1]);
      }
    }
    if constexpr (CL >= 2) {
      // Lane bit 3 (lanes l, l ^ 8: a rotation by 8 within rows of 16).
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t keep = b3 ? p[k + 4] : p[k], send = b3 ? p[k] : p[k + 4];
        p[k] = __builtin_elementwise_max(
            keep, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0x128, 0xf, 0xf, false));
      }
    }
#pragma unroll
    for (int k = 0; k < RV; ++k) run[t][k] = __builtin_elementwise_max(run[t][k], p[k]);
  };

  for (int x0 = 0; x0 < P + kPk; x0 += kPk) {
#pragma unroll
    for (int a = 0; a < kPk; ++a) {
      const int x = x0 + a;            // problem computed now; x - kPk is folded after it
      if (x >= P + kPk) break;
      float m = -INFINITY;
      if (x < P) {
        __builtin_amdgcn_sched_barrier(0);
        lds_wait_ge(&sm.q_ready, x + 1, ws, dead);
        // Q(x)'s slot is free again once every MFMA of the problem has read
        // it, or once its operands are in registers.
        const uint8_t *qs = &qsl.q[x % kQSlots][0];
        bf16x8 qreg[kQRegs ? kSteps : 1];
        if constexpr (kQRegs) {
#pragma unroll
          for (int st = 0; st < kSteps; ++st) qreg[st] = q_operand(qs, st);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          if (lane == 0) lds_inc(&sm.q_used[x % kQSlots]);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const f32x16 init = tile_init(t);
#pragma unroll
          for (int u = 0; u < UPT; ++u) {
            wait_unit();
            mfma_unit(ec[t], &ring.unit[wave][kc & (kRing - 1)][0], qreg, qs, u, init);
            // The MFMAs above have read the unit (their operands were
            // waited for): refill its slot.
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            ++kc;
            issue_next();
            __builtin_amdgcn_sched_barrier(0);   // keep the next unit's reads after the refill
          }
        }
        if constexpr (!kQRegs) {
          if (lane == 0) lds_inc(&sm.q_used[x % kQSlots]);   // (after the reads: lds_inc waits)
        }
        // Row max over the wave's keys (both halves), then e = 2^(x - m) in
        // place and the row sum (masked logits are -inf and give 0). The
        // lookahead keys keep their e: they are never stored.
        const float sl2 = kF8 ? s.scale_log2 * c.ks->v[x] : s.scale_log2;
        float mt = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) mt = fmaxf(mt, ec[t][i]);
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        m = mt * sl2;      // -inf when the wave has no key this row sees
        const float mz = m == -INFINITY ? 0.f : m;
        float z = 0.f;
        // (One tile at a time: left free, the scheduler computes every
        // tile's exponent arguments first and runs out of registers.)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float ev = __builtin_amdgcn_exp2f(__builtin_fmaf(ec[t][i], sl2, -mz));
            z += ev;
            ec[t][i] = ev;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        z += __shfl_xor(z, 32, 64);
        const int rs = x % kRedSlots;
        if (lane < 32) sm.red[rs][wave][r] = make_float2(m, z);
        // The last wave to finish the problem posts the block's partials.
        const int arrived =
            __builtin_amdgcn_readfirstlane(lane == 0 ? lds_inc(&sm.stats_cnt[rs]) : 0);
        if (arrived == kCompute * (x / kRedSlots + 1) - 1 && lane < kRows) {
          float M = -INFINITY, Z = 0.f;
#pragma unroll
          for (int w = 0; w < kCompute; ++w)
            stats_merge_lean(M, Z, sm.red[rs][w][lane].x, sm.red[rs][w][lane].y);
          // Twice: an ordinary store that the merge block of this die reads
          // from the die's L2, and a device-coherent one for a merge block
          // elsewhere.
          const int64_t at = cta_slot(x, c.cta) + lane;
          const uint64_t word = slot_word(lse_of(M, Z), ws.call_tag);
          ws.lslot[at] = word;
          __hip_atomic_store(ws.slot + at, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // Fold problem x - kPk (its lse is needed only now), then park x in
      // its slot.
      if (x >= kPk) {
        const int xf = x - kPk;
        lds_wait_ge(&sm.lse_ready[xf % kLseSlots], xf + 1, ws, dead);
        const float l2 = sm.lse[xf % kLseSlots][r];
        const float f = (row_ok && mref[a] != -INFINITY) ? __builtin_amdgcn_exp2f(mref[a] - l2) : 0.f;
        if (lane == 0) lds_inc(&sm.lse_used[xf % kLseSlots]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          fold_tile(a, t, f);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (x < P) {
#pragma unroll
        for (int t = 0; t < NT; ++t) park(ec[t], pk[a][t]);
        mref[a] = m;
      }
    }
  }

  // The rest of the reduction over the lane bits of the row (head r /
  // (32 / G) on the top bits, step r % (32 / G) on the bottom ones): first a
  // max over the head bits the fold left (G >= 8), then a sum over the step
  // bits (padding steps hold 0). Each level exchanges across one lane bit
  // (a swizzle within 32 lanes); it runs once per kernel.
  if constexpr (NT > 0) {
    float runf[NT][RV];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int k = 0; k < RV; ++k) runf[t][k] = __uint_as_float(run[t][k]);
    const int hb = __builtin_ctz(rs_h);          // lowest head bit
    constexpr int top = 4 - CL;                  // highest bit not reduced at fold time
    auto level = [&](auto bit_tag, bool use_max) {
      constexpr int B = decltype(bit_tag)::value;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int k = 0; k < RV; ++k) {
          const float o = __int_as_float(
              __builtin_amdgcn_ds_swizzle(__float_as_int(runf[t][k]), ((1 << B) << 10) | 0x1f));
          runf[t][k] = use_max ? fmaxf(runf[t][k], o) : runf[t][k] + o;
        }
    };
    auto both = [&](auto bit_tag) {
      constexpr int B = decltype(bit_tag)::value;
      if constexpr (B <= top) {
        if (B >= hb) level(bit_tag, true);
      }
    };
    auto steps = [&](auto bit_tag) {
      constexpr int B = decltype(bit_tag)::value;
      if constexpr (B <= top) {
        if (B < hb) level(bit_tag, false);
      }
    };
    both(std::integral_constant<int, 0>{});
    both(std::integral_constant<int, 1>{});
    both(std::integral_constant<int, 2>{});
    both(std::integral_constant<int, 3>{});
    both(std::integral_constant<int, 4>{});
    steps(std::integral_constant<int, 0>{});
    steps(std::integral_constant<int, 1>{});
    steps(std::integral_constant<int, 2>{});
    steps(std::integral_constant<int, 3>{});
    steps(std::integral_constant<int, 4>{});
    // Lanes whose reduced bits are all 0 hold the results of their keys:
    // acc index 8 b4 + 4 b3 + k for the compacted bits.
    const float inv_l = 1.f / (float)s.L;
    float *out = c.imp + c.tok0;
    const int low = r & ((1 << (5 - CL)) - 1);
    const int ibase = (CL >= 1 ? 8 * ((r >> 4) & 1) : 0) + (CL >= 2 ? 4 * ((r >> 3) & 1) : 0);
    if (low == 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int k = 0; k < RV; ++k) {
          const int key = w_key0 + t * t_stride + acc_row(ibase + k, half);
          if (key < N) out[key] = runf[t][k] * inv_l;
        }
    }
  }
}

template <int D, bool kF8, int kPk, int CL>
__global__ __launch_bounds__(kThreads, 1) void k_stream(AttnShape s, StreamTable tb,
                                                        int64_t total_keys,
                                                        const __bf16 *__restrict__ q,
                                                        const uint8_t *__restrict__ k,
                                                        float *__restrict__ imp, StreamWs ws,
                                                        KScales ks) {
  constexpr int kTPW = tpw_for_pk(kPk);              // tiles per compute wave
  using QL = UnitLayout<128>;
  constexpr int QU = D * 2 / 128;                    // Q units per problem (1 or 2)
  static_assert(QU * kUnitBytes <= kQSlotBytes, "Q slot too small");

  __shared__ Ring ring;
  __shared__ QSlots qsl;
  __shared__ Smem sm;
  const int cta = blockIdx.x;
  // The wave index is uniform across a wave; saying so keeps every value
  // derived from it in scalar registers and every branch on it scalar.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = s.n_layers * s.Hkv;
  if (cta >= tb.n_stream) {
    // Merge blocks, and idle blocks that only pad the merge blocks onto a
    // multiple of 8.
    if (cta >= tb.merge0) merge_block(s, tb, cta - tb.merge0, wave, lane, ws);
    return;
  }
  // The hand-off counters start at zero; the block's only barrier comes
  // before any load.
  if (tid == 0) {
    sm.q_ready = 0;
    for (int i = 0; i < kQSlots; ++i) sm.q_used[i] = 0;
    for (int i = 0; i < kRedSlots; ++i) sm.stats_cnt[i] = 0;
    for (int i = 0; i < kLseSlots; ++i) sm.lse_ready[i] = 0;
    for (int i = 0; i < kLseSlots; ++i) sm.lse_used[i] = 0;
    __hip_atomic_store(ws.hdr + 1, ws.call_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const int bb = cta_prompt(tb, cta), b = tb.p0 + bb;
  const int c_lo = tb.cta_off[bb], n_c = tb.cta_off[bb + 1] - c_lo, ci = cta - c_lo;
  const int N = tb.tok_off[bb + 1] - tb.tok_off[bb];
  const int NK = N + s.La;                                  // keys of the prompt
  const int64_t key0 = (int64_t)tb.tok_off[bb] + (int64_t)b * s.La;
  const int rows = s.L * s.G;
  bool dead = false;           // this wave gave up waiting (the call failed)

  if (wave == kCompute) {
    // ---------------- control wave ----------------
    // Q of problem y into slot y % 3 by direct loads; rows >= S * G read
    // past the resource and come back as zeros.
    const int64_t q_elems = (int64_t)s.n_layers * s.L * s.Hq * D;
    const __amdgpu_buffer_rsrc_t qr = rsrc(q + (int64_t)b * q_elems, (uint32_t)(q_elems * 2));
    uint32_t qoff[QL::IPU];   // per instruction: the lane's row and chunk within a problem's Q
    int qrow_j[QL::IPU], qrow_h[QL::IPU];
    const int rs_h = 32 / s.G;   // query row rr: head rr / (32 / G), step rr % (32 / G)
#pragma unroll
    for (int i = 0; i < QL::IPU; ++i) {
      const int rr = QL::KPI * i + lane / QL::SPK;
      const int c = (lane % QL::SPK) ^ QL::swz(rr);
      qrow_j[i] = rr % rs_h;
      qrow_h[i] = rr / rs_h;
      qoff[i] = (uint32_t)(16 * c);
    }
    auto issue_q = [&](int y) {
      const int l = y / s.Hkv, g = y - l * s.Hkv;
      uint8_t *dst = &qsl.q[y % kQSlots][0];
#pragma unroll
      for (int u = 0; u < QU; ++u)
#pragma unroll
        for (int i = 0; i < QL::IPU; ++i) {
          const uint32_t row_off =
              (uint32_t)((((int64_t)l * s.L + qrow_j[i]) * s.Hq + g * s.G + qrow_h[i]) * D * 2);
          const uint32_t vo = qrow_j[i] < s.L ? row_off + u * 128 + qoff[i] : kOob;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              qr, (__attribute__((address_space(3))) void *)(dst + u * kUnitBytes + 1024 * i), 16,
              vo, 0, 0, 0);
        }
    };
    // Problem y goes into the slot of y - 3 once every compute wave has read
    // that one. The wave's loads complete in order, and a Q load queues
    // behind the block's K stream (about 1.5 us), so Q loads go out between
    // problems, never between the polls of one: right after the lse of x is
    // staged, when every wave has finished x and the slot of Q(x + 3) is
    // free. Only when the compute waves may run further ahead than that
    // (lag > 2) does the poll loop top up as well.
    int q_issued = 0, q_marked = 0;
    auto top_up = [&]() {
      while (q_issued < P &&
             __builtin_amdgcn_readfirstlane(lds_get(&sm.q_used[q_issued % kQSlots])) >=
                 kCompute * (q_issued / kQSlots))
        issue_q(q_issued++);
    };
    top_up();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) lds_set(&sm.q_ready, q_issued);
    q_marked = q_issued;

    const unsigned dies = prompt_dies(c_lo, n_c);
    const int dlane = lane >> 3;
    const bool din = ((dies >> dlane) & 1u) != 0u;
    const uint32_t voff = dlane * kRows * (int)sizeof(uint64_t) + (lane & 7) * 32;
    auto poll = [&](int y) {
      const __amdgpu_buffer_rsrc_t rs =
          rsrc(ws.dslot + die_slot(y, bb, 0), kDies * kRows * (int)sizeof(uint64_t));
      return load_quad(rs, voff, 0);
    };
    // The die partials of the next kPoll problems are in flight together, so
    // a control wave that runs behind gets several problems' lse from one
    // round trip (a device-scope load takes ~1.5 us), not one. win[i] holds
    // problem x + i, polled when q_issued was wq[i]. Forms of three tiles per
    // wave only (long prompts; at 128K tokens 144 -> 140 us with four in
    // flight, eight no better): with fewer, shorter problems the extra polls
    // cost more than they bring (32K tokens: 68.1 -> 69.9 us).
    constexpr int kPoll = kPk <= 3 ? 4 : 1;
    Quad win[kPoll];
    int wq[kPoll];
#pragma unroll
    for (int i = 0; i < kPoll; ++i) {
      if (i < P) win[i] = poll(i);
      wq[i] = q_issued;
    }
    for (int x = 0; x < P; ++x) {
      // Die partials of x. Loads of one wave return in order: once a poll's
      // values are back, every Q load issued before it has landed too.
      Quad v[1] = {win[0]};
      const bool in[1] = {din};
      int q_round = wq[0];
      const uint64_t t0 = wall_clock64();
      for (;;) {
        const bool ok = !in[0] | quad_full(v[0], ws.call_tag);
        if (q_marked < q_round) {
          if (lane == 0) lds_set(&sm.q_ready, q_round);
          q_marked = q_round;
        }
        if (__all(ok) || dead) break;
        if (wall_clock64() - t0 > ws.wait_ticks) { timeout(ws, dead); break; }
        asm volatile("" ::: "memory");
        if (q_issued <= x + kPk) {    // the compute waves may need Q(x + kPk) now
          top_up();
        }
        q_round = q_issued;
        if (in[0] && !quad_full(v[0], ws.call_tag)) v[0] = poll(x);
      }
      const f32x4 lq = merge_quads(v, in);
      // The slot held the lse of x - 8: free once every compute wave folded it.
      lds_wait_ge(&sm.lse_used[x % kLseSlots], kCompute * (x / kLseSlots), ws, dead);
      if (lane < 8) *reinterpret_cast<f32x4 *>(&sm.lse[x % kLseSlots][4 * lane]) = lq;
      if (lane == 0) lds_set(&sm.lse_ready[x % kLseSlots], x + 1);
      top_up();
#pragma unroll
      for (int i = 0; i + 1 < kPoll; ++i) {
        win[i] = win[i + 1];
        wq[i] = wq[i + 1];
      }
      if (x + kPoll < P) win[kPoll - 1] = poll(x + kPoll);
      wq[kPoll - 1] = q_issued;
    }
    return;
  }

  // ---------------- compute waves ----------------
  // The prompt's keys in tiles of 32 (the last may be partial), dealt to its
  // blocks round-robin: block ci takes tiles ci, ci + n_c, ci + 2 n_c, ...
  // (within one tile of an even share), then split over the compute waves.
  // Wave w runs on SIMD w % 4, so waves w and w + 4 share one, and SIMD 3
  // holds only wave 3 besides the control wave. The tiles left over after
  // an even split go to waves 3, 0, 1, 2, 4, 5, 6 in that order, which
  // keeps the busiest SIMD's share lowest.
  const int ntiles = (NK + kTile - 1) / kTile;
  const int nt_blk = (ntiles - ci + n_c - 1) / n_c;
  const int base = nt_blk / kCompute, extra = nt_blk - base * kCompute;
  auto rank_of = [](int w) { return w == 3 ? 0 : w < 3 ? w + 1 : w; };
  auto tiles_of = [&](int w) { return base + (rank_of(w) < extra ? 1 : 0); };
  int w_t0 = 0;
  for (int w = 0; w < wave; ++w) w_t0 += tiles_of(w);
  const int nt = tiles_of(wave);   // this wave's tiles (<= kTPW)
  WaveCtx c;
  c.s = s;
  c.ws = ws;
  c.ks = &ks;
  c.k = k;
  c.imp = imp;
  c.total_keys = total_keys;
  c.key0 = key0;
  c.P = P;
  c.N = N;
  c.NK = NK;
  c.rows = rows;
  c.cta = cta;
  c.tok0 = tb.tok_off[bb];
  c.t_stride = n_c * kTile;
  c.w_key0 = (ci + n_c * w_t0) * kTile;
  c.wave = wave;
  c.lane = lane;
  // A tile is "full" (all keys are prompt keys, seen by every row) when it
  // ends by N; the wave's full tiles come first.
  int full_tiles = 0;
  while (full_tiles < nt && c.w_key0 + full_tiles * c.t_stride + kTile <= N) ++full_tiles;
  c.full_tiles = full_tiles;
  switch (nt) {
    case 0: compute_wave<D, kF8, kPk, CL, 0>(c, ring, qsl, sm, dead); break;
    case 1: compute_wave<D, kF8, kPk, CL, 1>(c, ring, qsl, sm, dead); break;
    case 2:
      if constexpr (kTPW >= 2) compute_wave<D, kF8, kPk, CL, 2>(c, ring, qsl, sm, dead);
      break;
    default:
      if constexpr (kTPW >= 3) compute_wave<D, kF8, kPk, CL, 3>(c, ring, qsl, sm, dead);
      break;
  }
}

struct DeviceInfo {
  int cus = 0;
  int occ = 0;        // blocks per CU of every kernel form (the least of them)
};

// Blocks per CU of every form of the kernel (the least of them).
template <int D, bool F8, int CL>
bool occupancy_cl(int *occ) {
  int a = 0, b = 0, c = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, k_stream<D, F8, pk_for_tpw(3, CL), CL>, kThreads, 0) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k_stream<D, F8, 4, CL>, kThreads, 0) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&c, k_stream<D, F8, 7, CL>, kThreads, 0) != hipSuccess)
    return false;
  *occ = std::min(*occ, std::min(a, std::min(b, c)));
  return true;
}
template <int D, bool F8>
bool occupancy(int *occ) {
  return occupancy_cl<D, F8, 0>(occ) && occupancy_cl<D, F8, 1>(occ) && occupancy_cl<D, F8, 2>(occ);
}

const DeviceInfo &device_info() {
  static DeviceInfo info[64];
  static bool done[64];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return info[0];
  std::lock_guard<std::mutex> lock(mu);
  if (!done[dev]) {
    DeviceInfo d;
    d.occ = 1 << 20;
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        !occupancy<128, false>(&d.occ) || !occupancy<64, false>(&d.occ) ||
        !occupancy<128, true>(&d.occ) || !occupancy<64, true>(&d.occ))
      d = DeviceInfo();
    info[dev] = d;
    done[dev] = true;
  }
  return info[dev];
}

// Split the batch into launches and give each prompt streaming blocks in
// proportion to its tiles (each block <= 21 tiles); the merge blocks follow
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
    int most = 1;
    for (int i = 0; i < B; ++i) {
      t.tok_off[i] = tok.tok_off[p0 + i];
      t.cta_off[i + 1] = t.cta_off[i] + need[i];
      most = std::max(most, (tiles[i] + need[i] - 1) / need[i]);
    }
    t.tok_off[B] = tok.tok_off[p0 + B];
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
int stream_ctas() {
  const DeviceInfo &d = device_info();
  if (d.occ < 1 || d.cus < 2 * kDies) return 0;
  return std::min(d.cus / kDies * kDies, kMaxCtas) - kDies;
}

size_t cta_region(const AttnShape &s) {
  return align_up((size_t)s.n_layers * s.Hkv * kMaxCtas * kRows * sizeof(uint64_t));
}
size_t die_region(const AttnShape &s) {
  return align_up((size_t)s.n_layers * s.Hkv * SP_MAX_PROMPTS * kDies * kRows * sizeof(uint64_t));
}

// The plan of a call, or false when the single pass does not take it.
bool plan_call(const AttnShape &s, const SegTable &tiles, Plan &plan) {
  if (!score_stream_supported(s)) return false;
  const int n_stream = stream_ctas();
  if (n_stream < 1) return false;
  // Lanes address K by 32-bit byte offsets from their prompt's first key row.
  const int64_t rowb = (int64_t)s.Hkv * s.d * (s.dtype == SP_DTYPE_BF16_FP8K ? 1 : 2);
  for (int b = 0; b < tiles.B; ++b) {
    const int64_t nk = (int64_t)tiles.tok_off[b + 1] - tiles.tok_off[b] + s.La;
    if (nk * rowb + rowb >= (int64_t)kOob) return false;
  }
  return make_plan(tiles, s.La, n_stream, plan);
}

}  // namespace

bool score_stream_supported(const AttnShape &s) {
  if (s.dtype != SP_DTYPE_BF16 && s.dtype != SP_DTYPE_BF16_FP8K) return false;
  if (s.row_pool > 1) return false;                   // pool-before-max: two-pass kernels
  if (s.G & (s.G - 1)) return false;                 // head groups of 2^k lanes
  if (!(s.scale_log2 > 0.f)) return false;           // row max from the logit max
  return true;
}

size_t score_stream_slot_bytes(const AttnShape &s) {
  if (!score_stream_supported(s)) return 0;
  return 2 * cta_region(s) + die_region(s);
}

bool score_stream_plan(const AttnShape &s, const SegTable &tiles, int *n_launches,
                       int32_t *prompt_launch) {
  static thread_local Plan plan;
  if (!plan_call(s, tiles, plan)) return false;
  *n_launches = plan.n_launch;
  if (prompt_launch)
    for (int li = 0; li < plan.n_launch; ++li)
      for (int i = 0; i < plan.t[li].B; ++i) prompt_launch[plan.t[li].p0 + i] = li;
  return true;
}

// Budget of each cross-block wait in wall-clock ticks (100 MHz): 2 s, or
// SP_SCORE_WAIT_US microseconds when that is set (up to about 3 hours).
uint64_t score_wait_ticks() {
  const char *e = getenv("SP_SCORE_WAIT_US");
  if (e && *e) {
    char *end = nullptr;
    const unsigned long long us = strtoull(e, &end, 10);
    if (end && *end == '\0') return std::min(us, 10000000000ull) * 100ull;
  }
  return 200000000ull;
}

hipError_t launch_score_stream(const AttnShape &s, const SegTable &tiles, const void *q,
                               const void *k, const KScales &ks, float *imp, void *ws,
                               hipStream_t st, bool *supported) {
  *supported = false;
  static thread_local Plan plan;
  if (!plan_call(s, tiles, plan)) return hipSuccess;
  *supported = true;
  StreamWs w;
  char *base = reinterpret_cast<char *>(ws);
  w.hdr = reinterpret_cast<uint32_t *>(base);
  base += kStatusBytes;
  w.slot = reinterpret_cast<uint64_t *>(base);
  w.lslot = reinterpret_cast<uint64_t *>(base + cta_region(s));
  w.dslot = reinterpret_cast<uint64_t *>(base + 2 * cta_region(s));
  w.wait_ticks = score_wait_ticks();
  const int64_t total_keys = (int64_t)tiles.tok_off[tiles.B] + (int64_t)tiles.B * tiles.L;
  const __bf16 *qp = reinterpret_cast<const __bf16 *>(q);
  const uint8_t *kp = reinterpret_cast<const uint8_t *>(k);
  const bool f8 = s.dtype == SP_DTYPE_BF16_FP8K;
  AttnShape sa = s;
  for (int li = 0; li < plan.n_launch; ++li) {
    w.call_tag = reserve_tags(1);
    // The most parked problems whose slots hold the tiles of the launch's
    // busiest compute wave.
    const int tpw = (plan.max_tiles[li] + kCompute - 1) / kCompute;
    // Head-max levels taken at fold time: lane bits 4 and 3 are head bits
    // for G >= 4, bit 4 for G = 2.
    const int cl = s.G >= 4 ? 2 : s.G == 2 ? 1 : 0;
    const int npk = pk_for_tpw(tpw, cl);
    auto pick = [&](auto d_tag, auto f8_tag) {
      constexpr int Dv = decltype(d_tag)::value;
      constexpr bool F8v = decltype(f8_tag)::value;
      auto by_pk = [&](auto cl_tag) {
        constexpr int C = decltype(cl_tag)::value;
        return npk == 7 ? k_stream<Dv, F8v, 7, C>
               : npk == 4 ? k_stream<Dv, F8v, 4, C>
                          : k_stream<Dv, F8v, pk_for_tpw(3, C), C>;
      };
      return cl == 2 ? by_pk(std::integral_constant<int, 2>{})
                     : cl == 1 ? by_pk(std::integral_constant<int, 1>{})
                               : by_pk(std::integral_constant<int, 0>{});
    };
    using D64 = std::integral_constant<int, 64>;
    using D128 = std::integral_constant<int, 128>;
    auto kern = s.d == 128 ? (f8 ? pick(D128{}, std::true_type{}) : pick(D128{}, std::false_type{}))
                           : (f8 ? pick(D64{}, std::true_type{}) : pick(D64{}, std::false_type{}));
    StreamTable tbl = plan.t[li];
    int64_t tk = total_keys;
    KScales kss = ks;
    void *args[] = {&sa, &tbl, &tk, &qp, &kp, &imp, &w, &kss};
    // An ordinary launch: the host has checked that the grid fits the device
    // with every block resident (one per CU). A cooperative launch would
    // guarantee it against other work on the device too, but costs ~11 us
    // more per call here; the bounded waits cover that case instead.
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(plan.grid[li]),
                                         dim3(kThreads), args, 0, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sp
