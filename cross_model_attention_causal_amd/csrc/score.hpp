// Transposed score tiles S^T = K Q^T on bf16 MFMA (32x32x16, fp32 accumulate).
//
// A wave owns 32 queries (one per lane column n = lane % 32; lanes n and n + 32
// hold the same query) and sweeps 64-key blocks. For key block c the wave holds
// two 32x32 tiles acc[kt]; element v of acc[kt] is key
//   64c + 32kt + 8(v/4) + 4(lane/32) + (v%4)
// of the lane's query. Each lane therefore sees 32 of the 64 keys of its query,
// in groups of 4 consecutive keys, and its partner lane (lane ^ 32) sees the rest:
// row reductions need one cross-lane exchange.
#pragma once
#include "common.hpp"

namespace cma {

template <int D>
struct QOperand {
  bf16x8 v[D / 16];
};

// Query operand (B of 32x32x16): lane holds Q[query][16ks + 8(lane/32) + e].
template <int D>
__device__ __forceinline__ void load_query(QOperand<D>& op, const uint16_t* qrow, bool valid) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (valid) x = ldg16(qrow + 16 * ks + 8 * half);
    op.v[ks] = as_bf16x8(x);
  }
}

// Scores of keys [key0, key0 + 64) (rows of K starting at kseq) against the
// wave's queries. Keys at or beyond nk give 0 (the caller masks them).
template <int D>
__device__ __forceinline__ void score_block(f32x16 acc[2], const QOperand<D>& qop,
                                            const uint16_t* __restrict__ kseq, int key0, int nk) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, half = lane >> 5;
  u32x4 a[2][D / 16];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = key0 + 32 * kt + m;
    const uint16_t* krow = kseq + (int64_t)key * D + 8 * half;
    const bool ok = key < nk;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (ok) x = ldg16(krow + 16 * ks);
      a[kt][ks] = x;
    }
  }
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    f32x16 c = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) c = mfma32(as_bf16x8(a[kt][ks]), qop.v[ks], c);
    acc[kt] = c;
  }
}

// Key index of element (kt, v) of a score block.
__device__ __forceinline__ int tile_key(int key0, int kt, int v) {
  const int half = (threadIdx.x & 63) >> 5;
  return key0 + 32 * kt + 8 * (v >> 2) + 4 * half + (v & 3);
}

// Scaled logits in log2 units with the sink bias and the causal mask applied:
// t = s * scale_l2 (+ bias_l2 on key 0); -inf where key > last (invisible).
__device__ __forceinline__ void logits_block(float t[32], const f32x16 acc[2], int key0, int last,
                                             float scale_l2, float bias_l2) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = tile_key(key0, kt, v);
      float x = acc[kt][v] * scale_l2;
      if (key == 0) x += bias_l2;
      t[kt * 16 + v] = (key <= last) ? x : -INFINITY;
    }
  }
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2f_fast(float x) { return __builtin_amdgcn_logf(x); }

// Online-softmax update of a query's running (max m, sum l) with one block of
// logits (log2 units). Both partner lanes end with identical values.
// Returns the block's partial sum relative to the new running max.
__device__ __forceinline__ float online_update(const float t[32], float& m, float& l) {
  float bm = -INFINITY;
#pragma unroll
  for (int e = 0; e < 32; ++e) bm = fmaxf(bm, t[e]);
  bm = fmaxf(bm, xor_lane(bm, 32));
  const float mn = fmaxf(m, bm);
  if (mn == -INFINITY) return 0.0f;
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) s += exp2f_fast(t[e] - mn);
  s += xor_lane(s, 32);
  l = l * exp2f_fast(m - mn) + s;
  m = mn;
  return s;
}

}  // namespace cma
