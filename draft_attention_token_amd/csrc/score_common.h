// Device helpers shared by the scoring kernels: MFMA operand fragments, the
// 32x32 logit tile, and the mapping of accumulator registers to (row, key).
#pragma once

#include "sp_internal.h"

namespace sp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x16 __attribute__((ext_vector_type(16)));

// One lane's share of a 32 x d operand for the 32x32 MFMA contraction over d.
//  bf16 (v_mfma_f32_32x32x16_bf16): d/16 k-steps; at step s the lane in half h
//    supplies d elements [16 s + 8 h, 16 s + 8 h + 8) as one 16-byte load.
//  fp32 (v_mfma_f32_32x32x2_f32): d/2 k-steps; at step s the lane in half h
//    supplies d element h * d/2 + s, so the lane reads d/2 contiguous floats.
// Q (A operand, row = lane % 32) and K (B operand, column = lane % 32) use
// the same element mapping, so every product pairs equal d indices.
template <typename T, int D> struct Frag;

template <int D> struct Frag<__bf16, D> {
  static constexpr int kSteps = D / 16;
  u32x4 v[kSteps];
  // Ordinary cached loads: one instruction reads 32 bytes of each of 32 key
  // rows, so four consecutive instructions share every 128-byte line; a
  // non-temporal hint lets the line go between them and costs a refetch each
  // time (K at ~3.3 instead of ~6 TB/s).
  __device__ __forceinline__ void load(const __bf16 *row, int half) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(row) + half;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) v[s] = p[2 * s];
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) v[s] = u32x4{0u, 0u, 0u, 0u};
  }
};

template <int D> struct Frag<float, D> {
  static constexpr int kSteps = D / 2;
  float v[kSteps];
  __device__ __forceinline__ void load(const float *row, int half) {
    const float4 *p = reinterpret_cast<const float4 *>(row + half * (D / 2));
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      float4 x = p[i];
      v[4 * i + 0] = x.x; v[4 * i + 1] = x.y; v[4 * i + 2] = x.z; v[4 * i + 3] = x.w;
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) v[s] = 0.f;
  }
};

// acc[r][c] = sum_d A[r][d] * B[c][d] for the wave's 32 rows and 32 keys.
template <int D>
__device__ __forceinline__ f32x16 mfma_tile(const Frag<__bf16, D> &a, const Frag<__bf16, D> &b) {
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < Frag<__bf16, D>::kSteps; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v[s]),
                                                 __builtin_bit_cast(bf16x8, b.v[s]), acc, 0, 0, 0);
  return acc;
}

template <int D>
__device__ __forceinline__ f32x16 mfma_tile(const Frag<float, D> &a, const Frag<float, D> &b) {
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < Frag<float, D>::kSteps; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[s], b.v[s], acc, 0, 0, 0);
  return acc;
}

// Row (query) held by accumulator register i of a lane in half h; the column
// (key) is lane % 32.
__device__ __forceinline__ constexpr int acc_row(int i, int half) {
  return 8 * (i >> 2) + 4 * half + (i & 3);
}

// Pointer to the d-vector of query row r = j * G + hh of (prompt b, layer l,
// KV group g) in q[B][layers][L][Hq][d] (L query steps, the prefill row
// included); rows >= L * G are padding.
template <typename T>
__device__ __forceinline__ const T *q_row_ptr(const T *q, const AttnShape &s, int b, int l, int g,
                                              int r) {
  const int j = r / s.G, hh = r - (r / s.G) * s.G;
  return q + ((((int64_t)b * s.n_layers + l) * s.L + j) * s.Hq + g * s.G + hh) * s.d;
}

// Pointer to key row `key` (global key index) of layer l, group g in
// k[layers][total_keys][Hkv][d].
template <typename T>
__device__ __forceinline__ const T *k_row_ptr(const T *k, const AttnShape &s, int64_t total_keys,
                                              int l, int64_t key, int g) {
  return k + (((int64_t)l * total_keys + key) * s.Hkv + g) * s.d;
}

__device__ __forceinline__ float wave_max32(float v) {
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum32(float v) {
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Merge of softmax partial statistics in base 2: (m, z) stands for
// sum_k 2^(x_k) = z * 2^m over some set of keys; m = -inf means empty.
__device__ __forceinline__ void stats_merge(float &M, float &Z, float m, float z) {
  if (m == -INFINITY) return;
  if (M == -INFINITY) { M = m; Z = z; return; }
  const float nm = fmaxf(M, m);
  Z = Z * exp2f(M - nm) + z * exp2f(m - nm);
  M = nm;
}

}  // namespace sp
