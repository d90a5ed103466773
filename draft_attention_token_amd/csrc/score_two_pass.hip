// Token importance, two-pass form: a statistics pass computes each softmax
// row's log-sum-exp over all keys it sees; a second pass recomputes the
// logits, turns them into probabilities, and reduces max over heads and
// layers and the mean over lookahead steps. K is read from HBM twice.
//
// Method: "SpecPrefill — Implementation Guide", How It Works / Token
// Importance (max over heads, then layers, then mean over lookahead steps),
// and "Speculative prefill" (llama.cpp pull request 27692), Approach
// steps 2-3. Causality: query j of a prompt sits at position N - pre + j
// and sees keys 0 .. N - pre + j (pre = 1 with the prefill row, the prompt's
// last row as step 0); only the N prompt columns receive importance.
#include "score_common.h"

namespace sp {
namespace {

// Logits of one 32-key tile of one (layer, KV group) for the lane; returns
// the tile context through the out-parameters.
struct TileCtx {
  int b;          // prompt
  int64_t N;      // prompt tokens
  int64_t nkeys;  // N + L keys
  int64_t key0;   // global key row of the prompt's key 0
  int64_t kl;     // local key index of this lane's column
};

__device__ __forceinline__ TileCtx tile_ctx(const SegTable &tiles, int t, int col) {
  TileCtx c;
  c.b = seg_of(tiles, t);
  c.N = tiles.tok_off[c.b + 1] - tiles.tok_off[c.b];
  c.nkeys = c.N + tiles.L;
  c.key0 = tiles.tok_off[c.b] + (int64_t)c.b * tiles.L;
  c.kl = (int64_t)(t - tiles.unit_off[c.b]) * kTile + col;
  return c;
}

template <typename T, int D>
__device__ __forceinline__ f32x16 tile_logits(const AttnShape &s, const TileCtx &c,
                                              int64_t total_keys, const T *q, const T *k, int l,
                                              int g, int lane) {
  const int half = lane >> 5, r = lane & 31;
  Frag<T, D> a, bk;
  if (r < s.L * s.G) a.load(q_row_ptr(q, s, c.b, l, g, r), half); else a.zero();
  if (c.kl < c.nkeys) bk.load(k_row_ptr(k, s, total_keys, l, c.key0 + c.kl, g), half); else bk.zero();
  return mfma_tile<D>(a, bk);
}

// The Q rows of (prompt b, layer l, KV group g) into LDS rows, 16 bytes per
// thread and step (rows >= L * G are left alone: no lane reads them).
template <typename T, int D>
__device__ __forceinline__ void stage_q_rows(T (*qs)[D + 16 / sizeof(T)], const AttnShape &s,
                                             const T *q, int b, int l, int g, int tid, int nthr) {
  constexpr int kVecs = D * (int)sizeof(T) / 16;   // 16-byte vectors per row
  const int rows = s.L * s.G;
  for (int i = tid; i < rows * kVecs; i += nthr) {
    const int row = i / kVecs, v = i - row * kVecs;
    reinterpret_cast<u32x4 *>(&qs[row][0])[v] =
        reinterpret_cast<const u32x4 *>(q_row_ptr(q, s, b, l, g, row))[v];
  }
}

// Pass 1: per (tile, layer, group), the base-2 max and sum of 2^(logit - max)
// of each of the 32 rows over the tile's visible keys. One wave per (tile,
// problem), four waves (four consecutive tiles) per block; the block stages
// the problem's Q rows in LDS once (a wave whose tile lies in another prompt
// reads its own). K is the MFMA A operand, so a lane holds one query row
// (lane % 32) and 16 of the tile's keys: each row's max and sum reduce inside
// the lane plus one swap of wave halves.
constexpr int kStatsWaves = 4;
template <typename T, int D>
__global__ __launch_bounds__(64 * kStatsWaves) void k_stats(AttnShape s, SegTable tiles,
                                                            int64_t total_keys, int total_tiles,
                                                            const T *__restrict__ q,
                                                            const T *__restrict__ k,
                                                            float2 *__restrict__ part) {
  __shared__ __align__(16) T qs[kRows][D + 16 / sizeof(T)];   // padded rows
  const int t = blockIdx.x * kStatsWaves + (int)(threadIdx.x >> 6), prob = blockIdx.y;
  const int l = prob / s.Hkv, g = prob - l * s.Hkv;
  const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
  const int rows = s.L * s.G;
  const int b0 = seg_of(tiles, blockIdx.x * kStatsWaves);
  stage_q_rows<T, D>(qs, s, q, b0, l, g, threadIdx.x, 64 * kStatsWaves);
  __syncthreads();
  if (t >= total_tiles) return;
  const TileCtx c = tile_ctx(tiles, t, col);       // c.kl: the key this lane loads
  Frag<T, D> a, bk;
  if (col >= rows) a.zero();
  else if (c.b == b0) a.load(&qs[col][0], half);
  else a.load(q_row_ptr(q, s, c.b, l, g, col), half);
  if (c.kl < c.nkeys) bk.load(k_row_ptr(k, s, total_keys, l, c.key0 + c.kl, g), half); else bk.zero();
  const f32x16 acc = mfma_tile<D>(bk, a);          // acc[i]: key acc_row(i, half), row col
  const int j = col / s.G;
  const int64_t kbase = c.kl - col;                // the tile's first key
  float x[16], m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t key = kbase + acc_row(i, half);
    const bool vis = col < rows && key < c.nkeys && key <= c.N - s.pre + j;
    x[i] = vis ? acc[i] * s.scale_log2 : -INFINITY;
    m = fmaxf(m, x[i]);
  }
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) z += x[i] == -INFINITY ? 0.f : exp2f(x[i] - m);
  z += __shfl_xor(z, 32, 64);
  if (half == 0) part[((int64_t)prob * total_tiles + t) * kRows + col] = make_float2(m, z);
}

// Combine the tile statistics of each (prompt, layer, group, row) in a fixed
// order: lse2 = m + log2(z) (base-2 log-sum-exp of the row's logits). 32
// contiguous tile ranges per row, eight loads in flight per thread, then the
// ranges merged in order.
constexpr int kLseParts = 32;
__global__ __launch_bounds__(kLseParts * kRows) void k_lse(SegTable tiles, int n_prob,
                                                           int total_tiles,
                                                           const float2 *__restrict__ part,
                                                           float *__restrict__ lse,
                                                           uint32_t *__restrict__ hdr,
                                                           uint32_t call_tag) {
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) hdr[1] = call_tag;   // no waits here
  __shared__ float2 sm[kLseParts][kRows];
  const int b = blockIdx.x, prob = blockIdx.y;
  const int row = threadIdx.x & 31, p = threadIdx.x >> 5;
  const int t0 = tiles.unit_off[b], t1 = tiles.unit_off[b + 1];
  const int per = (t1 - t0 + kLseParts - 1) / kLseParts;
  const int ta = t0 + p * per, tb = min(t1, ta + per);
  const float2 *src = part + (int64_t)prob * total_tiles * kRows + row;
  float M = -INFINITY, Z = 0.f;
  for (int t = ta; t < tb; t += 8) {
    float2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = t + u < tb ? src[(int64_t)(t + u) * kRows] : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u) stats_merge(M, Z, v[u].x, v[u].y);
  }
  sm[p][row] = make_float2(M, Z);
  __syncthreads();
  if (p == 0) {
    for (int i = 1; i < kLseParts; ++i) stats_merge(M, Z, sm[i][row].x, sm[i][row].y);
    lse[((int64_t)b * n_prob + prob) * kRows + row] = (Z > 0.f) ? M + log2f(Z) : INFINITY;
  }
}

// Pass 2: per tile, all layers and groups, dealt to the block's waves; p =
// 2^(x - lse2); the step-max over (layer, head) lives in LDS as ordered uint
// (p >= 0, so the float bits order like the values); then the mean over
// steps. Several waves per tile keep short prompts (few tiles) from running
// every problem of a tile one after another.
constexpr int kScoreWaves = 8;
template <typename T, int D>
__global__ __launch_bounds__(64 * kScoreWaves) void k_score(AttnShape s, SegTable tiles,
                                                            int64_t total_keys,
                                                            const T *__restrict__ q,
                                                            const T *__restrict__ k,
                                                            const float *__restrict__ lse,
                                                            float *__restrict__ imp) {
  __shared__ unsigned smax[kRows][kTile];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  for (int i = threadIdx.x; i < kRows * kTile; i += 64 * kScoreWaves) (&smax[0][0])[i] = 0u;
  __syncthreads();
  const TileCtx c = tile_ctx(tiles, t, col);
  const int n_prob = s.n_layers * s.Hkv, rows = s.L * s.G;
  const bool prompt_key = c.kl < c.N;
  for (int prob = wave; prob < n_prob; prob += kScoreWaves) {
    const int l = prob / s.Hkv, g = prob - l * s.Hkv;
    const f32x16 acc = tile_logits<T, D>(s, c, total_keys, q, k, l, g, lane);
    const float *lrow = lse + ((int64_t)c.b * n_prob + prob) * kRows;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = acc_row(i, half);
      if (row < rows && prompt_key) {
        const float p = exp2f(acc[i] * s.scale_log2 - lrow[row]);
        atomicMax(&smax[row / s.G][col], __float_as_uint(p));
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 32 && prompt_key) {
    float acc = 0.f;
    for (int j = 0; j < s.L; ++j) acc += __uint_as_float(smax[j][col]);
    imp[tiles.tok_off[c.b] + c.kl] = acc / (float)s.L;
  }
}

// Pass 2, pool-before-max form ("Speculative prefill", Approach step 3, read
// with the smoothing first): every (layer, head) probability row is pooled
// over its prompt keys (centred window of W = 2 r + 1 keys, divided by the
// number of prompt keys inside it) before the max over heads and layers.
// A block owns one 32-key output tile at k0 and computes the probabilities
// of keys [k0 - 16, k0 + 48) as two logit tiles (the window's reach is at
// most 16 keys each side) and parks them in LDS; a lane then reads one row's
// 48 probabilities around its 16 output keys into registers and adds each
// window afresh (no running sum that subtracts, which would cancel near a
// large probability).
// Blocks take tiles die by die (block i runs on die i % 8 and gets the i / 8-th
// tile of that die's contiguous share), so neighbouring tiles, which read each
// other's halo keys, meet in the same L2. The tile's problems are dealt to
// the block's kW waves, each with its own probability buffer: four for
// short batches (few tiles, whose problems would otherwise run one after
// another), one for long ones (more blocks per CU in flight instead).
constexpr int kPooledManyTiles = 2048;   // batches this long take one wave per tile
template <typename T, int D, int kW>
__global__ __launch_bounds__(64 * kW) void k_score_pooled(
    AttnShape s, SegTable tiles, int64_t total_keys, int total_tiles, const T *__restrict__ q,
    const T *__restrict__ k, const float *__restrict__ lse, float *__restrict__ imp) {
  __shared__ float pvs[kW][kPoolSpan][kRows + 1];   // [key - (k0 - kPoolHalo)][row]
  __shared__ unsigned smax[kRows][kTile + 1];   // padded: rows fall in different banks
  const int per = (total_tiles + 7) / 8;
  const int t = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (t >= total_tiles) return;
  const int b = seg_of(tiles, t);
  const int N = tiles.tok_off[b + 1] - tiles.tok_off[b];
  const int k0 = (t - tiles.unit_off[b]) * kTile;   // first output key (prompt-local)
  if (k0 >= N) return;                               // a tile of lookahead keys only
  const int64_t key0 = tiles.tok_off[b] + (int64_t)b * tiles.L;
  const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  float(*pv)[kRows + 1] = pvs[wave];
  for (int i = threadIdx.x; i < kRows * kTile; i += 64 * kW) (&smax[0][0])[i] = 0u;
  const int n_prob = s.n_layers * s.Hkv, rows = s.L * s.G;
  const int r = (s.row_pool - 1) / 2;
  // The lane's 16 output keys for row `col` in the pooling step.
  const int c0 = 16 * half;
  // With 2^k heads per group, the max over a step's heads is taken across its
  // G lanes and kept in registers (per lane: its step, its 16 keys) until the
  // end; other group sizes take it in LDS with atomics.
  const bool pow2 = (s.G & (s.G - 1)) == 0;
  float run[kTile / 2];
#pragma unroll
  for (int c = 0; c < kTile / 2; ++c) run[c] = 0.f;
  // Every wave runs the same number of rounds (the block barriers below);
  // a wave without a problem in a round only takes part in them.
  const int rounds = (n_prob + kW - 1) / kW;
  for (int round = 0; round < rounds; ++round) {
    const int prob = round * kW + wave;
    const bool active = prob < n_prob;
    const int l = active ? prob / s.Hkv : 0, g = active ? prob - l * s.Hkv : 0;
    Frag<T, D> a;
    if (col < rows) a.load(q_row_ptr(q, s, b, l, g, col), half); else a.zero();
    const float *lrow = lse + ((int64_t)b * n_prob + (active ? prob : 0)) * kRows;
    float lr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = acc_row(i, half);
      lr[i] = row < rows ? lrow[row] : INFINITY;
    }
#pragma unroll
    for (int u = 0; u < kPoolSpan / kTile; ++u) {
      const int kl = k0 - kPoolHalo + kTile * u + col;   // this lane's key column
      const bool need = active && kl >= 0 && kl < N && kl >= k0 - r && kl < k0 + kTile + r;
      Frag<T, D> bk;
      if (need) bk.load(k_row_ptr(k, s, total_keys, l, key0 + kl, g), half); else bk.zero();
      const f32x16 acc = mfma_tile<D>(a, bk);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = need ? exp2f(acc[i] * s.scale_log2 - lr[i]) : 0.f;   // 0 for padding rows
        pv[kTile * u + col][acc_row(i, half)] = p;
      }
    }
    __syncthreads();
    float pc[kTile / 2];   // pooled probabilities of the lane's row and 16 keys
#pragma unroll
    for (int c = 0; c < kTile / 2; ++c) pc[c] = 0.f;
    if (active && col < rows) {
      // The row's probabilities of keys k0 + c0 - 16 .. k0 + c0 + 31 (pv rows
      // c0 .. c0 + 47), all read up front; each window sum then adds its
      // terms in key order, zeros outside the window.
      float v[kTile / 2 + 2 * kPoolHalo];
#pragma unroll
      for (int x = 0; x < kTile / 2 + 2 * kPoolHalo; ++x) v[x] = pv[c0 + x][col];
      auto emit = [&](int c, float w) {
        const int kk = k0 + c0 + c;
        const int lo = max(0, kk - r), hi = min(N - 1, kk + r);
        pc[c] = kk < N ? w / (float)(hi - lo + 1) : 0.f;
      };
      if (r == kDefaultPoolRadius) {
        // The default width: the window is known at compile time.
#pragma unroll
        for (int c = 0; c < kTile / 2; ++c) {
          float w = 0.f;
#pragma unroll
          for (int o = -kDefaultPoolRadius; o <= kDefaultPoolRadius; ++o) w += v[c + kPoolHalo + o];
          emit(c, w);
        }
      } else {
#pragma unroll
        for (int c = 0; c < kTile / 2; ++c) {
          float w = 0.f;
#pragma unroll
          for (int o = -kPoolHalo; o <= kPoolHalo; ++o)
            w += (o >= -r && o <= r) ? v[c + kPoolHalo + o] : 0.f;
          emit(c, w);
        }
      }
    }
    if (pow2) {
      for (int m = 1; m < s.G; m <<= 1)
#pragma unroll
        for (int c = 0; c < kTile / 2; ++c) pc[c] = fmaxf(pc[c], __shfl_xor(pc[c], m, 64));
#pragma unroll
      for (int c = 0; c < kTile / 2; ++c) run[c] = fmaxf(run[c], pc[c]);
    } else if (active && col < rows) {
#pragma unroll
      for (int c = 0; c < kTile / 2; ++c)
        if (k0 + c0 + c < N) atomicMax(&smax[col / s.G][c0 + c], __float_as_uint(pc[c]));
    }
    __syncthreads();
  }
  if (pow2 && col < rows && col % s.G == 0) {
    // One lane per step and half; the block's waves meet here.
#pragma unroll
    for (int c = 0; c < kTile / 2; ++c) atomicMax(&smax[col / s.G][c0 + c], __float_as_uint(run[c]));
  }
  __syncthreads();
  if (threadIdx.x < kTile && k0 + lane < N) {
    float acc = 0.f;
    for (int j = 0; j < s.L; ++j) acc += __uint_as_float(smax[j][lane]);
    imp[tiles.tok_off[b] + k0 + lane] = acc / (float)s.L;
  }
}

template <typename T, int D>
hipError_t run(const AttnShape &s, const SegTable &tiles, int total_tiles, const void *q,
               const void *k, float *imp, uint32_t *hdr, void *region, hipStream_t st) {
  const int n_prob = s.n_layers * s.Hkv;
  const int64_t total_keys = tiles.tok_off[tiles.B] + (int64_t)tiles.B * tiles.L;
  float2 *part = reinterpret_cast<float2 *>(region);
  float *lse = reinterpret_cast<float *>(reinterpret_cast<char *>(part) +
                                         align_up((size_t)n_prob * total_tiles * kRows * sizeof(float2)));
  hipLaunchKernelGGL((k_stats<T, D>), dim3((total_tiles + kStatsWaves - 1) / kStatsWaves, n_prob),
                     dim3(64 * kStatsWaves), 0, st, s, tiles, total_keys, total_tiles,
                     (const T *)q, (const T *)k, part);
  hipLaunchKernelGGL(k_lse, dim3(tiles.B, n_prob), dim3(kLseParts * kRows), 0, st, tiles, n_prob,
                     total_tiles, part, lse, hdr, reserve_tags(1));
  if (s.row_pool > 1) {
    const dim3 grid((total_tiles + 7) / 8 * 8);
    if (total_tiles < kPooledManyTiles)
      hipLaunchKernelGGL((k_score_pooled<T, D, 4>), grid, dim3(64 * 4), 0, st, s, tiles, total_keys,
                         total_tiles, (const T *)q, (const T *)k, lse, imp);
    else
      hipLaunchKernelGGL((k_score_pooled<T, D, 1>), grid, dim3(64), 0, st, s, tiles, total_keys,
                         total_tiles, (const T *)q, (const T *)k, lse, imp);
  } else {
    hipLaunchKernelGGL((k_score<T, D>), dim3(total_tiles), dim3(64 * kScoreWaves), 0, st, s, tiles,
                       total_keys, (const T *)q, (const T *)k, lse, imp);
  }
  return hipGetLastError();
}

}  // namespace

size_t score_two_pass_region_bytes(const AttnShape &s, int B, int total_tiles) {
  const size_t n_prob = (size_t)s.n_layers * s.Hkv;
  return align_up(n_prob * total_tiles * kRows * sizeof(float2)) +
         align_up((size_t)B * n_prob * kRows * sizeof(float));
}

hipError_t launch_score_two_pass(const AttnShape &s, const SegTable &tiles, int total_tiles,
                                 const void *q, const void *k, float *imp, uint32_t *hdr,
                                 void *region, hipStream_t st) {
  if (s.dtype == SP_DTYPE_BF16) {
    if (s.d == 128) return run<__bf16, 128>(s, tiles, total_tiles, q, k, imp, hdr, region, st);
    return run<__bf16, 64>(s, tiles, total_tiles, q, k, imp, hdr, region, st);
  }
  if (s.d == 128) return run<float, 128>(s, tiles, total_tiles, q, k, imp, hdr, region, st);
  return run<float, 64>(s, tiles, total_tiles, q, k, imp, hdr, region, st);
}

}  // namespace sp
