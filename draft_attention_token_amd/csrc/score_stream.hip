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
//  * Persistent grid, one block per CU, all blocks co-resident (cooperative
//    launch). A block owns <= 18 contiguous 32-key tiles of one prompt for
//    the whole kernel (prompt keys and lookahead keys alike).
//  * The work is a sequence of problems (layer l, KV group g), each with
//    L * G <= 32 query rows (step j, head-in-group hh), padded to 32.
//  * Six compute waves per block, <= 3 tiles each. Per problem a wave
//    computes logits with 32x32x16 bf16 MFMA, K as the A operand (MFMA row =
//    key) and Q as the B operand (MFMA column = query row): a lane holds one
//    query row and 16 keys of each tile, so a row's max and sum over the
//    wave's keys reduce inside the lane plus one swap of wave halves. As soon as a
//    tile's MFMAs have consumed its K registers, the wave refills them with
//    the next problem's tile: the K stream never waits for synchronisation.
//  * One control wave per block does all cross-block work, so no compute
//    wave ever waits on a fence or an atomic (on this hardware, waiting on
//    any memory operation also waits on every load issued before it, which
//    would drain the K prefetch). Per problem it merges the compute waves'
//    (m, z), posts it, and takes a ticket; the last block of the prompt to
//    arrive merges every block's (m, z) in block order and publishes the row
//    lse. It also stages the next problem's Q and an earlier problem's lse in
//    LDS for the compute waves.
//  * The compute waves fold problem i - 2 while working on problem i: they
//    park e in LDS (two problem slots) and later turn it into probabilities
//    p = e * 2^(m_tile - lse), kept as a running max per (row, key) in
//    registers (max over layers and KV groups). Two problems of lag give the
//    ticket, merge and publish a full problem's time to land. The row
//    statistics are accumulated tile by tile (online max and rescaled sum),
//    and each tile's e is relative to the running max at that tile, so only
//    one tile's logits are live at a time.
//  * Finally: max over the G heads of a step (lanes of a group), mean over
//    the L steps (a fixed tree across groups of lanes), store.
// Every wait is bounded (about 2 s); on time-out the kernel records it in the
// workspace status word and runs to completion, so the grid always drains.
// No cache-wide fence is used: cross-block slots are relaxed agent-scope
// atomics that validate themselves (see StreamWs).
#include <string.h>

#include <algorithm>

#include "score_common.h"

namespace sp {
namespace {

constexpr int kCompute = 6;                       // compute waves per block
constexpr int kThreads = (kCompute + 1) * 64;     // plus one control wave
constexpr int kTPW = 3;                           // tiles per compute wave
constexpr int kTilesPerCta = kCompute * kTPW;     // 18
constexpr int kLag = 2;                           // problems between logits and fold
constexpr int kStatusWords = kStatusBytes / sizeof(int);
constexpr uint64_t kWaitTicks = 200000000ull;     // wall clock runs at 100 MHz: 2 s
constexpr int kQPad = 8;                          // bf16 padding per staged Q row
constexpr int kMaxCtas = 1024;                    // blocks per launch (one per CU)

struct StreamTable {
  int32_t B;        // prompts in this launch
  int32_t p0;       // global index of the first one
  int32_t tok_off[SP_MAX_PROMPTS + 1];   // global token offsets of prompts p0 .. p0 + B
  int32_t cta_off[SP_MAX_PROMPTS + 1];   // block prefix within this launch
};

// Cross-block data lives in 64-bit slots written and read with relaxed
// agent-scope atomics (coherent across the chip's L2s without cache-wide
// fences), and every slot tells by itself whether it has been written, so no
// ordering between different slots is needed:
//   part slot = (m, z) float bits; all-zero bits mean "not yet written" (a
//     written slot has z > 0, or m = -inf for a row with no visible keys);
//   lse slot  = float bits | 1 << 32 once published.
// The launcher zeroes status, tickets, lse and part before each launch.
struct StreamWs {
  int *status;                 // [kStatusWords]; status[0] != 0: a wait timed out
  unsigned long long *lse;     // [B_total][P][32] tagged base-2 lse of each row
  unsigned long long *part;    // [P][n_cta][32] block (m, z)
};

template <int D>
struct Smem {
  f32x4 eprev[kLag][kCompute][kTPW][4][64];   // parked e values (16-byte slots per lane)
  __bf16 q[kRows][D + kQPad];                 // staged Q rows of the next problem
  float2 red[2][kCompute][kRows];             // per-wave (m, z) of a problem
  float lse[kRows];                           // staged lse of the problem being folded
};

__device__ __forceinline__ int cta_prompt(const StreamTable &t, int c) {
  int lo = 0, hi = t.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t.cta_off[mid] <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ unsigned long long pack2(float m, float z) {
  return (unsigned long long)__float_as_uint(m) | ((unsigned long long)__float_as_uint(z) << 32);
}

__device__ __forceinline__ void timeout(int *status) {
  __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Reducer of one row of one problem: merge the row's (m, z) from every block
// of the prompt in a fixed order (lane l takes blocks l, l + 64, ...; lanes
// then merge in a fixed binary tree, lower lane first), and publish lse. A
// slot that is still empty (its block has not posted yet) is read again.
__device__ void reduce_row(const StreamWs &ws, int prob, int row, int n_cta, int c_lo, int n_c,
                           int b, int P, int lane) {
  const unsigned long long *base = ws.part + ((int64_t)prob * n_cta + c_lo) * kRows + row;
  constexpr int kPer = kMaxCtas / 64;
  unsigned long long v[kPer];
  const uint64_t t0 = wall_clock64();
  for (;;) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = u * 64 + lane;
      v[u] = c < n_c ? __hip_atomic_load(base + (int64_t)c * kRows, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT)
                     : 1ull;
    }
    bool ok = true;
#pragma unroll
    for (int u = 0; u < kPer; ++u) ok &= v[u] != 0ull;
    if (__all(ok)) break;
    if (wall_clock64() - t0 > kWaitTicks) { timeout(ws.status); break; }
    __builtin_amdgcn_s_sleep(1);
  }
  float M = -INFINITY, Z = 0.f;
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (u * 64 + lane < n_c)
      stats_merge(M, Z, __uint_as_float((unsigned)v[u]), __uint_as_float((unsigned)(v[u] >> 32)));
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float mo = __shfl_xor(M, off, 64), zo = __shfl_xor(Z, off, 64);
    if (lane & off) {           // lower lane's value first
      float a = mo, bz = zo;
      stats_merge(a, bz, M, Z);
      M = a; Z = bz;
    } else {
      stats_merge(M, Z, mo, zo);
    }
  }
  if (lane == 0) {
    const float l2 = Z > 0.f ? M + log2f(Z) : INFINITY;
    __hip_atomic_store(ws.lse + ((int64_t)b * P + prob) * kRows + row,
                       (1ull << 32) | __float_as_uint(l2), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Block that reduces row `row` of problem `prob`: spread over the prompt's
// blocks and rotated from problem to problem.
__device__ __forceinline__ int reducer_of(int prob, int row, int n_c) {
  return (row * 37 + prob * 11) % n_c;
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void k_stream(AttnShape s, StreamTable tb,
                                                        int64_t total_keys, int n_cta,
                                                        const __bf16 *__restrict__ q,
                                                        const __bf16 *__restrict__ k,
                                                        float *__restrict__ imp, StreamWs ws) {
  __shared__ Smem<D> sm;
  const int cta = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, r = lane & 31;
  const bool control = wave == kCompute;
  const int bb = cta_prompt(tb, cta), b = tb.p0 + bb;
  const int c_lo = tb.cta_off[bb], n_c = tb.cta_off[bb + 1] - c_lo, ci = cta - c_lo;
  const int N = tb.tok_off[bb + 1] - tb.tok_off[bb];
  const int NK = N + s.L;                                   // keys of the prompt
  const int tiles = (NK + kTile - 1) / kTile;
  const int ta = (int)((int64_t)tiles * ci / n_c);
  const int nt = (int)((int64_t)tiles * (ci + 1) / n_c) - ta;
  const int w_t0 = ta + (nt * wave) / kCompute;
  const int w_nt = control ? 0 : ta + (nt * (wave + 1)) / kCompute - w_t0;
  const int64_t key0 = (int64_t)tb.tok_off[bb] + (int64_t)b * s.L;
  const int P = s.n_layers * s.Hkv;
  const int rows = s.L * s.G;
  const bool row_ok = r < rows;
  const int jr = row_ok ? r / s.G : 0;

  if (control) {
    // ---------------- control wave: all cross-block work ----------------
    // Per iteration (after the second barrier): post this problem's block
    // statistics; start reading the previous problem's lse (needed at the
    // next iteration); reduce the rows of this problem this block is the
    // reducer of; load the Q of problem it + 2. Between the two barriers it
    // only writes LDS from registers.
    QRegs<D> qn;
    float lse_next = 0.f;
    load_q(qn, s, q, b, 0, lane);
    store_q(sm, qn, lane);
    if (P > 1) load_q(qn, s, q, b, 1, lane);
    __syncthreads();
    for (int it = 0; it < P + kLag; ++it) {
      __syncthreads();   // B1: wave statistics of problem it are in LDS
      if (it >= kLag && lane < kRows) sm.lse[lane] = lse_next;
      if (it + 1 < P) store_q(sm, qn, lane);
      __syncthreads();   // B2: lse of problem it - kLag and Q of problem it + 1 are in LDS
      if (it < P && lane < kRows) {
        float M = -INFINITY, Z = 0.f;
#pragma unroll
        for (int w = 0; w < kCompute; ++w)
          stats_merge(M, Z, sm.red[it & 1][w][lane].x, sm.red[it & 1][w][lane].y);
        __hip_atomic_store(ws.part + ((int64_t)it * n_cta + cta) * kRows + lane, pack2(M, Z),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      // Previous problem's lse: published by its reducers one period ago.
      const int pf = it + 1 - kLag;
      unsigned long long lv = 0ull;
      const unsigned long long *lslot =
          ws.lse + ((int64_t)b * P + (pf >= 0 ? pf : 0)) * kRows + (lane & 31);
      const bool need = pf >= 0 && pf < P && lane < s.L * s.G;   // padding rows: no lse
      if (need) lv = __hip_atomic_load(lslot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (it < P) {
        for (int row = 0; row < kRows; ++row)
          if (row < s.L * s.G && reducer_of(it, row, n_c) == ci)
            reduce_row(ws, it, row, n_cta, c_lo, n_c, b, P, lane);
      }
      if (it + 2 < P) load_q(qn, s, q, b, it + 2, lane);
      if (pf >= 0 && pf < P) {
        if (need) {
          const uint64_t t0 = wall_clock64();
          while (!(lv >> 32)) {
            if (wall_clock64() - t0 > kWaitTicks) { timeout(ws.status); break; }
            __builtin_amdgcn_s_sleep(1);
            lv = __hip_atomic_load(lslot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        lse_next = __uint_as_float((unsigned)lv);
      }
    }
    return;
  }

  // ---------------- compute waves ----------------
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

  // Loads are unconditional (addresses clamped into the prompt; keys outside
  // the wave's tiles are masked later), which keeps the compiler's wait
  // counts exact: a tile's MFMAs wait for that tile's loads only.
  auto load_k = [&](int prob, int t) {
    const int l = prob / s.Hkv, g = prob - l * s.Hkv;
    const int key = min((w_t0 + t) * kTile + r, NK - 1);
    kf[t].load(k_row_ptr(k, s, total_keys, l, key0 + key, g), half);
  };

#pragma unroll
  for (int t = 0; t < kTPW; ++t) load_k(0, t);
  __syncthreads();

  // Q operand rows in LDS: lane r reads its row's 8 bf16 of each k-step.
  const u32x4 *qs = reinterpret_cast<const u32x4 *>(&sm.q[r][0]) + half;

  for (int it = 0; it < P + kLag; ++it) {
    const int slot = it % kLag;
#pragma unroll
    for (int a = kLag; a > 0; --a)
#pragma unroll
      for (int t = 0; t < kTPW; ++t) mref[a][t] = mref[a - 1][t];
    if (it < P) {
      // Tile by tile: logits, online max / sum; e relative to the running
      // max at that tile (kept in mref).
      float m = -INFINITY, z = 0.f;
#pragma unroll
      for (int t = 0; t < kTPW; ++t) {
        f32x16 x = {};
#pragma unroll
        for (int st = 0; st < Frag<__bf16, D>::kSteps; ++st)
          x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[t].v[st]),
                                                     __builtin_bit_cast(bf16x8, qs[2 * st]), x, 0,
                                                     0, 0);
        load_k(it + 1 < P ? it + 1 : it, t);   // the last problem reloads its own tile
        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = (w_t0 + t) * kTile + acc_row(i, half);
          const bool ok = row_ok && t < w_nt && key <= N + jr;   // causal; implies key < NK
          x[i] = ok ? x[i] * s.scale_log2 : -INFINITY;
          mt = fmaxf(mt, x[i]);
        }
        const float mn = fmaxf(m, mt);
        if (mn != -INFINITY) {
          z = m == -INFINITY ? 0.f : z * __builtin_amdgcn_exp2f(m - mn);
          m = mn;
        }
        mref[0][t] = m;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = x[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[i] - m);
          z += e;
          const int key = (w_t0 + t) * kTile + acc_row(i, half);
          E[t][i] = key < N ? e : 0.f;    // lookahead keys get no importance
        }
      }
      // Merge the two wave halves (same row, different keys).
      const float mo = __shfl_xor(m, 32, 64), zo = __shfl_xor(z, 32, 64);
      float M = m, Z = z;
      if (half) { M = mo; Z = zo; stats_merge(M, Z, m, z); }
      else stats_merge(M, Z, mo, zo);
      if (lane < 32) sm.red[it & 1][wave][r] = make_float2(M, Z);
    }
    __syncthreads();   // B1
    __syncthreads();   // B2
    if (it >= kLag) {
      // Fold problem it - kLag: p = e * 2^(m_tile - lse), max into run;
      // then its LDS slot takes this problem's e (same lane, in order).
      const float l2 = sm.lse[r];
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

  // Max over the G heads of each step (lanes j*G .. j*G+G-1), then the mean
  // over the steps (groups of lanes; padding rows hold 0).
  {
#pragma unroll
    for (int t = 0; t < kTPW; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = run[t][i];
        for (int off = 1; off < s.G; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
        for (int off = s.G; off < kRows; off <<= 1) v += __shfl_xor(v, off, 64);
        run[t][i] = v;
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
}

__global__ void k_zero(u32x4 *p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

struct DeviceInfo {
  int cus = 0;
  int occ64 = 0, occ128 = 0;
  bool coop = false;
};

const DeviceInfo &device_info() {
  static DeviceInfo info[64];
  static bool done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return info[0];
  if (!done[dev]) {
    DeviceInfo d;
    int coop = 0;
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.occ64, k_stream<64>, kThreads, 0) !=
            hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.occ128, k_stream<128>, kThreads, 0) !=
            hipSuccess)
      d = DeviceInfo();
    d.coop = coop != 0;
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
  if (!d.coop || occ < 1 || d.cus < 1) return 0;
  return d.cus;
}


StreamWs carve(void *ws, int B, int P, size_t *zero_bytes) {
  char *p = reinterpret_cast<char *>(ws);
  StreamWs w;
  w.status = reinterpret_cast<int *>(p);
  p += align_up(kStatusWords * sizeof(int));
  w.lse = reinterpret_cast<unsigned long long *>(p);
  p += align_up((size_t)B * P * kRows * sizeof(unsigned long long));
  w.part = reinterpret_cast<unsigned long long *>(p);
  p += align_up((size_t)P * kMaxCtas * kRows * sizeof(unsigned long long));
  *zero_bytes = (size_t)(p - reinterpret_cast<char *>(ws));
  return w;
}

}  // namespace

bool score_stream_supported(const AttnShape &s, int B, int total_tiles) {
  (void)B;
  (void)total_tiles;
  if (s.dtype != SP_DTYPE_BF16) return false;
  if (s.G & (s.G - 1)) return false;                 // head groups of 2^k lanes
  return true;
}

size_t score_stream_ws(const AttnShape &s, int B, int total_tiles) {
  (void)total_tiles;
  const int P = s.n_layers * s.Hkv;
  return align_up(kStatusWords * sizeof(int)) +
         align_up((size_t)B * P * kRows * sizeof(unsigned long long)) +
         align_up((size_t)P * kMaxCtas * kRows * sizeof(unsigned long long));
}

hipError_t launch_score_stream(const AttnShape &s, const SegTable &tiles, int total_tiles,
                               const void *q, const void *k, float *imp, void *ws,
                               size_t ws_bytes, hipStream_t st, bool *supported) {
  *supported = false;
  if (!score_stream_supported(s, tiles.B, total_tiles)) return hipSuccess;
  const int n_cta = stream_ctas(s);
  if (n_cta < 1 || n_cta > kMaxCtas) return hipSuccess;
  static thread_local Plan plan;
  if (!make_plan(tiles, s.L, n_cta, plan)) return hipSuccess;
  if (ws_bytes < score_stream_ws(s, tiles.B, total_tiles)) return hipSuccess;
  *supported = true;
  const int P = s.n_layers * s.Hkv;
  size_t zb = 0;
  StreamWs w = carve(ws, tiles.B, P, &zb);
  // Only the part slots the launches use need clearing, not all kMaxCtas.
  const size_t used = (size_t)((char *)(w.part + (size_t)P * n_cta * kRows) - (char *)w.status);
  (void)zb;
  const int nzero = (int)(used / sizeof(u32x4));
  hipLaunchKernelGGL(k_zero, dim3(std::min(1024, (nzero + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<u32x4 *>(w.status), nzero);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total_keys = (int64_t)tiles.tok_off[tiles.B] + (int64_t)tiles.B * tiles.L;
  const __bf16 *qp = reinterpret_cast<const __bf16 *>(q);
  const __bf16 *kp = reinterpret_cast<const __bf16 *>(k);
  for (int li = 0; li < plan.n_launch; ++li) {
    StreamTable tb = plan.t[li];
    int ncta = n_cta;
    AttnShape sh = s;
    void *args[] = {(void *)&sh, (void *)&tb, (void *)&total_keys, (void *)&ncta, (void *)&qp,
                    (void *)&kp, (void *)&imp, (void *)&w};
    const void *fn = s.d == 128 ? (const void *)k_stream<128> : (const void *)k_stream<64>;
    e = hipLaunchCooperativeKernel(fn, dim3(plan.grid[li]), dim3(kThreads), args, 0, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sp
