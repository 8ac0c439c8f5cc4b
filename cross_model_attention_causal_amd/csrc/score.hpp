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
#include <type_traits>

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

// As load_query for a row index that may lie past the sequence end: every lane
// loads (row `safe`, an existing row) and invalid lanes then take zeros, so no
// load sits under a divergent branch.
template <int D>
__device__ __forceinline__ void load_query_clamped(QOperand<D>& op, const uint16_t* qrow_safe, bool valid) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 x = ldg16(qrow_safe + 16 * ks + 8 * half);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = valid ? x[e] : 0u;
    op.v[ks] = as_bf16x8(x);
  }
}

// As load_query_clamped without the zeroing: every lane takes the row it points
// at (a row past the sequence end points at an existing row), for callers that
// never use the results of such rows. Nothing consumes the loaded registers
// here, so the loads stay in flight until the operand's first use.
template <int D>
__device__ __forceinline__ void load_query_rows(QOperand<D>& op, const uint16_t* qrow_safe) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) op.v[ks] = as_bf16x8(ldg16(qrow_safe + 16 * ks + 8 * half));
}

// One 64-key block of K as the A operand of 32x32x16 (lane holds key
// key0 + 32kt + lane % 32, features 16ks + 8(lane/32) + e). Held in registers so
// that the next block can be fetched while the current one is multiplied.
template <int D>
struct KTile {
  u32x4 a[2][D / 16];
};

// Load keys [key0, key0 + 64) (rows of K starting at kseq); keys at or beyond nk
// read as zero (the caller masks them).
template <int D>
__device__ __forceinline__ void load_k(KTile<D>& kt_, const uint16_t* __restrict__ kseq, int key0, int nk) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, half = lane >> 5;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = key0 + 32 * kt + m;
    const uint16_t* krow = kseq + (int64_t)key * D + 8 * half;
    const bool ok = key < nk;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (ok) x = ldg16(krow + 16 * ks);
      kt_.a[kt][ks] = x;
    }
  }
}

template <int D>
__device__ __forceinline__ void mma_k(f32x16 acc[2], const KTile<D>& kt_, const QOperand<D>& qop) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    f32x16 c = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) c = mfma32(as_bf16x8(kt_.a[kt][ks]), qop.v[ks], c);
    acc[kt] = c;
  }
}

// Scores of keys [key0, key0 + 64) against the wave's queries (load + multiply).
template <int D>
__device__ __forceinline__ void score_block(f32x16 acc[2], const QOperand<D>& qop,
                                            const uint16_t* __restrict__ kseq, int key0, int nk) {
  KTile<D> k;
  load_k<D>(k, kseq, key0, nk);
  mma_k<D>(acc, k, qop);
}

// ---- K staged in LDS
// A stage holds 4 key blocks x 64 keys x 64 features (one half of D = 128, or
// all of D = 64): 128 bytes per key as 8 chunks of 16 bytes, chunk ch of key m
// in slot ch ^ ((m >> 1) & 7), so that the 16 lanes of one read pass (keys
// m..m+15, one chunk column) hit 16 distinct 4-bank groups. Block b occupies
// bytes [8192 b, 8192 (b + 1)) of the stage. The two query tiles of a block-row
// read the same stage, so K crosses L2 -> LDS once per workgroup, in 1 KB runs.
constexpr int kStageBlockBytes = 64 * 128;
constexpr int kStageBytes = 4 * kStageBlockBytes;

// Copy of feature half FH of the 4 blocks whose first keys are key0[b], in two
// parts so that the global loads can be in flight while the stage in use is
// read: kstage_load fetches into registers, kstage_store writes them to a stage.
// 512 threads: wave w moves keys 8w .. 8w + 7 of every block, one 16-byte chunk
// per lane and block, so each load reads 8 whole 128-byte lines and each LDS
// write fills 1 KB contiguously. Keys at or beyond nk are clamped to nk - 1:
// finite values the caller masks.
struct KStageRegs {
  u32x4 x[4];
};

template <int D, int FH>
__device__ __forceinline__ void kstage_load(KStageRegs& rg, const uint16_t* __restrict__ kseq, int nk,
                                            const int key0[4]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = 8 * wave + (lane >> 3), s = lane & 7;
  const int ch = s ^ ((m >> 1) & 7);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int key = min(key0[b] + m, nk - 1);
    rg.x[b] = ldg16(kseq + (int64_t)key * D + 64 * FH + 8 * ch);
  }
}

__device__ __forceinline__ void kstage_store(uint8_t* stage, const KStageRegs& rg) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int b = 0; b < 4; ++b) *reinterpret_cast<u32x4*>(stage + b * kStageBlockBytes + 16 * tid) = rg.x[b];
}

// acc[kt] += K_half(block at blk) x Q_half^T for feature half FH (A operand from
// the stage, B operand = the wave's queries). The two kt chains are interleaved.
template <int D, int FH>
__device__ __forceinline__ void kstage_mma(f32x16 acc[2], const uint8_t* blk, const QOperand<D>& qop) {
  const int lane = threadIdx.x & 63;
  const int hl = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 x[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int m = 32 * kt + (lane & 31);
      const int ch = 2 * ks + hl;
      x[kt] = *reinterpret_cast<const u32x4*>(blk + m * 128 + 16 * (ch ^ ((m >> 1) & 7)));
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) acc[kt] = mfma32(as_bf16x8(x[kt]), qop.v[4 * FH + ks], acc[kt]);
  }
}

// Per-sub-step K pipeline (attention maps, block statistics and extraction). A
// sub-step is one feature half
// of a round of 4 key blocks. Two LDS stages alternate; the global loads of
// sub-step u + 2 are in flight (in registers) while sub-step u is computed, and
// sub-step u + 1 (loaded one iteration earlier) is written to the other stage at
// the end of the iteration, before the barrier that publishes it. The count of
// sub-steps run is rounded up to even, so a body can be called once for the round
// just past the end: it must do nothing there (key0_of clamps its key blocks).
template <int D, typename Key0, typename Body>
__device__ __forceinline__ void kstage_pipeline(uint8_t* stage, const uint16_t* __restrict__ kseq, int nk,
                                                int rounds, Key0 key0_of, Body body) {
  constexpr int FH = D / 64;
  const int nsub = rounds * FH;
  const int ne = (nsub + 1) & ~1;  // sub-steps run (see below)
  auto load = [&](KStageRegs& rg, int u) {
    int key0[4];
    const int k = u / FH;
#pragma unroll
    for (int b = 0; b < 4; ++b) key0[b] = key0_of(4 * k + b);
    if (FH == 1 || u % FH == 0) kstage_load<D, 0>(rg, kseq, nk, key0);
    else kstage_load<D, FH - 1>(rg, kseq, nk, key0);
  };
  auto run = [&](int u) {
    const uint8_t* buf = stage + (u & 1) * kStageBytes;
    if (FH == 1 || u % FH == 0) body(u / FH, buf, std::integral_constant<int, 0>{});
    else body(u / FH, buf, std::integral_constant<int, FH - 1>{});
  };
  // iteration u: regs `mine` held sub-step u (already in LDS) and now fetch u + 2;
  // regs `next` hold sub-step u + 1. Past the end the indices are clamped: the
  // extra loads are harmless and keep the control flow (and so the compiler's
  // wait counting) straight.
  auto iter = [&](KStageRegs& mine, KStageRegs& next, int u) {
    load(mine, min(u + 2, ne - 1));
    run(u);
    kstage_store(stage + ((u + 1) & 1) * kStageBytes, next);
    barrier_lds();
  };
  if (nsub == 0) return;
  // An even count of sub-steps (the body takes one past the end as empty), so
  // that the loop has a single exit: with an exit between the two copies of the
  // step, the compiler's waits at the loop head assume the first copy's loads may
  // still be in flight there and drain them.
  KStageRegs r0, r1;
  load(r0, 0);
  load(r1, 1);
  kstage_store(stage, r0);
  barrier_lds();
  for (int u = 0; u < ne; u += 2) {
    iter(r0, r1, u);
    iter(r1, r0, u + 1);
  }
}

// Whole-block K pipeline: a sub-step stages two key blocks with all their
// features (block j in slots j * D / 64 .. + D / 64 - 1, one 64-feature half per
// slot; with D = 64 slots 2 and 3 repeat slots 0 and 1), so that a wave finishes
// one block per sub-step. Depth 2, as kstage_pipeline: the loads of sub-step
// u + 2 are in flight while sub-step u is computed.
template <int D>
__device__ __forceinline__ void kstage_load2(KStageRegs& rg, const uint16_t* __restrict__ kseq, int nk, int key0a,
                                             int key0b) {
  constexpr int FHN = D / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = 8 * wave + (lane >> 3), s = lane & 7;
  const int ch = s ^ ((m >> 1) & 7);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int blk = FHN == 2 ? (b >> 1) : (b & 1), fh = FHN == 2 ? (b & 1) : 0;
    const int key = min((blk ? key0b : key0a) + m, nk - 1);
    rg.x[b] = ldg16(kseq + (int64_t)key * D + 64 * fh + 8 * ch);
  }
}

struct NoPrologue {
  __device__ void operator()() const {}
};

// `pro` runs once after the first loads are issued, before the loop (a body that
// stores uses it to issue as many non-writing stores as one sub-step, so that the
// compiler's waits at the loop head count an iteration's stores on every path).
template <int D, typename Key0, typename Body, typename Pro = NoPrologue>
__device__ __forceinline__ void kstage2_pipeline(uint8_t* stage, const uint16_t* __restrict__ kseq, int nk, int nsub,
                                                 Key0 key0_of, Body body, Pro pro = Pro{}) {
  const int ne = (nsub + 1) & ~1;  // an even count, as in kstage_pipeline
  auto load = [&](KStageRegs& rg, int u) { kstage_load2<D>(rg, kseq, nk, key0_of(2 * u), key0_of(2 * u + 1)); };
  auto iter = [&](KStageRegs& mine, KStageRegs& next, int u) {
    load(mine, min(u + 2, ne - 1));  // clamped past the end: harmless, keeps the control flow straight
    body(u, stage + (u & 1) * kStageBytes);
    kstage_store(stage + ((u + 1) & 1) * kStageBytes, next);
    barrier_lds();
  };
  if (nsub == 0) return;
  // sub-step 1 is fetched first: on the path into the loop, the operations after
  // it (sub-step 0's loads, `pro`, the first iteration's own) then number at
  // least those of an iteration, so the first wait for it leaves earlier stores
  // in flight
  KStageRegs r0, r1;
  load(r1, 1);
  load(r0, 0);
  pro();
  kstage_store(stage, r0);
  barrier_lds();
  for (int u = 0; u < ne; u += 2) {
    iter(r0, r1, u);
    iter(r1, r0, u + 1);
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

// As logits_block, in place in the accumulators.
__device__ __forceinline__ void logits_inplace(f32x16 acc[2], int key0, int last, float scale_l2, float bias_l2) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = tile_key(key0, kt, v);
      float x = acc[kt][v] * scale_l2;
      if (key == 0) x += bias_l2;
      acc[kt][v] = (key <= last) ? x : -INFINITY;
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
  bm = pair32_max(bm);
  const float mn = fmaxf(m, bm);
  if (mn == -INFINITY) return 0.0f;
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) s += exp2f_fast(t[e] - mn);
  s = pair32_add(s);
  l = l * exp2f_fast(m - mn) + s;
  m = mn;
  return s;
}

// As online_update, on logits held in the accumulator registers.
__device__ __forceinline__ float online_update_acc(const f32x16 t[2], float& m, float& l) {
  float bm = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int v = 0; v < 16; ++v) bm = vmax(bm, t[kt][v]);
  bm = pair32_max(bm);
  const float mn = fmaxf(m, bm);
  if (mn == -INFINITY) return 0.0f;
  float s = 0.0f;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += exp2f_fast(t[kt][v] - mn);
  s = pair32_add(s);
  l = l * exp2f_fast(m - mn) + s;
  m = mn;
  return s;
}

// Scheduling hints for one wave's instruction stream: `n` instructions of a kind
// next (kinds as the compiler's scheduler numbers them).
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100;
#define CMA_SCHED(kind, n) __builtin_amdgcn_sched_group_barrier((kind), (n), 0)

// Online update for a block that needs no mask and no sink bias (every key is
// visible to every query of the wave and none is key 0), taking the raw scores.
// Requires scale_l2 > 0, so that the largest raw score gives the largest logit;
// the exponent is one fused multiply-add, 2^(s * scale_l2 - max).
__device__ __forceinline__ float online_update_raw(const f32x16 acc[2], float scale_l2, float& m, float& l) {
  // IEEE maximum (NaN-propagating) needs no quieting of the matrix products'
  // results and fuses into three-operand instructions
  float b4[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) b4[u] = vmax(acc[0][u], acc[0][u + 4]);
#pragma unroll
  for (int v = 8; v < 16; ++v) b4[v & 3] = vmax(b4[v & 3], acc[0][v]);
#pragma unroll
  for (int v = 0; v < 16; ++v) b4[v & 3] = vmax(b4[v & 3], acc[1][v]);
  float bm = vmax(vmax(b4[0], b4[1]), vmax(b4[2], b4[3]));
  bm = pair32_max(bm) * scale_l2;
  const float mn = fmaxf(m, bm);
  float s4[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) s4[v] = exp2f_fast(fmaf(acc[0][v], scale_l2, -mn));
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int v = 4 * (1 - kt); v < 16; ++v) s4[v & 3] += exp2f_fast(fmaf(acc[kt][v], scale_l2, -mn));
  float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  s = pair32_add(s);
  l = l * exp2f_fast(m - mn) + s;
  m = mn;
  return s;
}

// The products of one block (K staged at blk, both feature halves for D = 128)
// into acc_new, beside the lean online update of the previous block (acc_old),
// in one straight stretch of code whose schedule alternates operand reads,
// products and the update's vector instructions: the matrix core and the vector
// unit then work at the same time within one wave. Returns the update's
// partial sum.
template <int D>
__device__ __forceinline__ float mma_beside_update(f32x16 acc_new[2], const uint8_t* blk, const QOperand<D>& qop,
                                                   const f32x16 acc_old[2], float scale_l2, float& m, float& l) {
  acc_new[0] = acc_new[1] = f32x16{};
  kstage_mma<D, 0>(acc_new, blk, qop);
  if constexpr (D == 128) kstage_mma<D, 1>(acc_new, blk + kStageBlockBytes, qop);
  const float part = online_update_raw(acc_old, scale_l2, m, l);
  constexpr int NM = D / 8;  // products (32x32x16) per block
#pragma unroll
  for (int t = 0; t < NM; ++t) {
    CMA_SCHED(kSchedDsRead, 1);
    CMA_SCHED(kSchedMfma, 1);
    CMA_SCHED(kSchedValu, 6);
  }
  return part;
}

}  // namespace cma
