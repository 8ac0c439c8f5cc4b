// Causal attention probability maps (GLIDE II-B; materialised as IAM Method 4
// requires). Writing the map is the HBM cost of this stage. Four kernels, chosen
// per launch:
//  * k_attn_rows: one query row per sequence (decode), keys read once;
//  * k_attn_maps_short: every sequence has at most 512 keys; a persistent
//    workgroup keeps a (sequence, head)'s K in LDS and forms each block-row's
//    softmax in one pass from scores held in registers;
//  * k_attn_maps: longer sequences, two sweeps per 64-query block-row (online
//    max and normaliser, then recompute and write exp(s - max) / sum);
//    recomputing QK^T is cheaper than a round trip of the map;
//  * k_attn_maps_f32: fp32 inputs (the reference path), one row per workgroup.
#include "kernels.hpp"
#include "score.hpp"

namespace cma {

// Store 4 consecutive map entries of one row, starting at element index `idx`
// of the output, writing only the first `cnt` (0..4) of them.
template <bool BF16>
__device__ __forceinline__ void store4(void* out, int64_t idx, const float p[4], int cnt) {
  if (BF16) {
    uint16_t* o = reinterpret_cast<uint16_t*>(out) + idx;
    if (cnt == 4 && (idx & 3) == 0) {
      u32x2 w = {pack2bf(p[0], p[1]), pack2bf(p[2], p[3])};
      *reinterpret_cast<u32x2*>(o) = w;
    } else {
      for (int e = 0; e < cnt; ++e) o[e] = f2bf(p[e]);
    }
  } else {
    float* o = reinterpret_cast<float*>(out) + idx;
    if (cnt == 4 && (idx & 3) == 0) {
      *reinterpret_cast<f32x4*>(o) = f32x4{p[0], p[1], p[2], p[3]};
    } else {
      for (int e = 0; e < cnt; ++e) o[e] = p[e];
    }
  }
}

// 1-D grid of 8 * ceil(n_seqs * n_heads / 8) * n_rb workgroups, dealt to the 8
// XCDs round robin: workgroup b runs on XCD b % 8 and takes slot b / 8 there; the
// n_rb consecutive slots of a (sequence, head) unit are its block-rows, longest
// first, so the block-rows that re-read one K run on one XCD and share its L2.
// 512 threads = 8 waves: wave w owns
// queries 32 (w & 1) .. + 31 of the block-row and key blocks 4k + (w >> 1) of
// each round of the staged K (kstage_pipeline: 4 key blocks x one feature half
// per sub-step, the loads of the sub-step after next in flight). Dynamic LDS:
// the two K stages.
constexpr int kTileRow = 36;  // dwords per row of a wave's bf16 output tile (64 keys + pad)

template <int D, bool PACKED, bool OUT_BF16>
__global__ __launch_bounds__(512) void k_attn_maps(AttnMapsArgs a) {
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  uint8_t* stage = reinterpret_cast<uint8_t*>(dyn);
  __shared__ __attribute__((aligned(16))) uint32_t wtile[OUT_BF16 ? 8 : 1][OUT_BF16 ? 32 * kTileRow : 1];
  const int slot = (int)(blockIdx.x >> 3);
  const int unit = 8 * (slot / a.n_rb) + (int)(blockIdx.x & 7);
  if (unit >= a.vl.n_seqs * a.n_heads) return;
  const int s = unit % a.vl.n_seqs, h = unit / a.vl.n_seqs;
  const int r = a.n_rb - 1 - slot % a.n_rb;
  const int32_t nq = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
  if (!seq_ok(a.vl, s, nq, nk) || 64 * r >= nq) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int qt = wave & 1, kp = wave >> 1;
  const int i = 64 * r + 32 * qt + (lane & 31);
  const bool valid = i < nq;
  const int last = nk - nq + i;  // last visible key of this query
  const int rowmax = min(64 * r + 63, nq - 1);
  const int cmax = (nk - nq + rowmax) >> 6;  // last key block of the block-row
  // last key block of the wave's queries (past it every key is masked for them)
  const int cmax_t = (nk - nq + min(64 * r + 32 * qt + 31, nq - 1)) >> 6;

  const uint16_t* qrow = a.q + ((int64_t)h * a.vl.total_q + cu_q_of(a.vl, s) + min(i, nq - 1)) * D;
  const uint16_t* kseq = a.k + ((int64_t)h * a.vl.total_k + cu_k_of(a.vl, s)) * D;
  const float scale_l2 = ld_const(a.scale + h) * kLog2e;
  const float bias_l2 = a.bias ? ld_const(a.bias + h) * kLog2e : 0.0f;

  QOperand<D> qop;
  load_query_clamped<D>(qop, qrow, valid);

  f32x16 acc[2];
  float m = -INFINITY, l = 0.0f;
  // Blocks with every key visible to every query of the wave and no sink key
  // take the lean path on raw scores (needs a positive scale).
  const bool raw_ok = scale_l2 > 0.0f;
  const int first_last = nk - nq + 64 * r + 32 * qt;  // last key of the wave's first query
  auto lean = [&](int c) { return raw_ok && c != 0 && 64 * c + 63 <= first_last; };
  auto key0_of = [&](int c) { return 64 * min(c, cmax); };
  // Sweep 1: running max and sum.
  kstage_pipeline<D>(stage, kseq, nk, (cmax + 4) / 4, key0_of, [&](int k, const uint8_t* buf, auto fh) {
    constexpr int FH = decltype(fh)::value;
    const int c = 4 * k + kp;
    if (c > cmax_t) return;
    if (FH == 0) acc[0] = acc[1] = f32x16{};
    kstage_mma<D, FH>(acc, buf + kp * kStageBlockBytes, qop);
    if (FH != D / 64 - 1) return;
    if (lean(c)) {
      online_update_raw(acc, scale_l2, m, l);
    } else {
      logits_inplace(acc, 64 * c, valid ? last : -1, scale_l2, bias_l2);
      online_update_acc(acc, m, l);
    }
  });

  __shared__ float sm[4][64], sl[4][64];
  if (lane < 32) {
    sm[kp][32 * qt + lane] = m;
    sl[kp][32 * qt + lane] = l;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][32 * qt + (lane & 31)]);
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = sm[w][32 * qt + (lane & 31)];
    if (mw != -INFINITY) L += sl[w][32 * qt + (lane & 31)] * exp2f_fast(mw - M);
  }
  const float lse = M + log2f_fast(L);

  const int64_t base0 = (int64_t)h * a.head_stride + map_seq_off(a.vl, s, PACKED);
  const int64_t base = base0 + map_row_off(i, nq, nk, PACKED);
  const int wend = PACKED ? last + 1 : nk;  // entries of this row that exist in the layout
  const int cend = PACKED ? cmax : (nk - 1) >> 6;
  const int half = lane >> 5;
  // Sweep 2: recompute and write p = 2^(logit - lse); dense rows also get the
  // zeros of blocks past the diagonal.
  kstage_pipeline<D>(stage, kseq, nk, (cend + 4) / 4, key0_of, [&](int k, const uint8_t* buf, auto fh) {
    constexpr int FH = decltype(fh)::value;
    const int c = 4 * k + kp;
    if (c > cend) return;
    const bool comp = c <= cmax_t;
    if (comp) {
      if (FH == 0) acc[0] = acc[1] = f32x16{};
      kstage_mma<D, FH>(acc, buf + kp * kStageBlockBytes, qop);
    }
    if (FH != D / 64 - 1) return;
    if (comp) {
      if (lean(c)) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[kt][v] = exp2f_fast(fmaf(acc[kt][v], scale_l2, -lse));
      } else {
        logits_inplace(acc, 64 * c, valid ? last : -1, scale_l2, bias_l2);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[kt][v] = exp2f_fast(acc[kt][v] - lse);
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) acc[kt] = f32x16{};
    }
    if constexpr (OUT_BF16) {
      // Through the wave's LDS tile, so that the global stores run along rows:
      // lane (query q, half) puts its 4-key groups at tile row q, then each pass
      // writes two rows (32 lanes per row) of the block's segment [64c, 64c + len)
      // with 4-byte stores on the row's own alignment (a packed row may start at
      // any element) and 2-byte stores for a leading or trailing odd entry.
      uint32_t* tw = wtile[wave];
      wave_lds_fence();  // the previous block's reads of the tile come first
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 w = {pack2bf(acc[kt][4 * g], acc[kt][4 * g + 1]), pack2bf(acc[kt][4 * g + 2], acc[kt][4 * g + 3])};
          *reinterpret_cast<u32x2*>(&tw[(lane & 31) * kTileRow + 16 * kt + 4 * g + 2 * half]) = w;
        }
      wave_lds_fence();  // rows are read by other lanes
      const int kl = lane & 31, rsel = lane >> 5;
      for (int p2 = 0; p2 < 16; ++p2) {
        const int qq = 2 * p2 + rsel;
        const int iq = 64 * r + 32 * qt + qq;
        const int len = iq < nq ? min(64, (PACKED ? nk - nq + iq + 1 : nk) - 64 * c) : 0;
        if (len <= 0) continue;
        uint16_t* out = reinterpret_cast<uint16_t*>(a.maps) + base0 + map_row_off(iq, nq, nk, PACKED) + 64 * c;
        const int sh = (int)((reinterpret_cast<uintptr_t>(out) >> 1) & 1), j0 = sh + 2 * kl;  // 4-byte phase
        const uint16_t* trow = reinterpret_cast<const uint16_t*>(&tw[qq * kTileRow]);
        if (j0 + 1 < len) *reinterpret_cast<uint32_t*>(out + j0) = (uint32_t)trow[j0] | ((uint32_t)trow[j0 + 1] << 16);
        else if (j0 < len) out[j0] = trow[j0];
        if (sh && kl == 0) out[0] = trow[0];
      }
    } else {
      if (!valid) return;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int key0 = 64 * c + 32 * kt + 8 * g + 4 * half;
          const float p[4] = {acc[kt][4 * g], acc[kt][4 * g + 1], acc[kt][4 * g + 2], acc[kt][4 * g + 3]};
          const int cnt = max(0, min(4, wend - key0));
          if (cnt > 0) store4<OUT_BF16>(a.maps, base + key0, p, cnt);
        }
      }
    }
  });
}

// ---- Short sequences (every sequence has at most 512 keys): one pass.
// A persistent workgroup (one per CU) takes (sequence, head) units round robin
// and walks each unit's block-rows in order. The unit's K stays resident in LDS
// (up to 8 blocks in the staged layout, block c in slots c * D / 64 ..): block c
// goes in just before the first block-row that sees it, so K crosses HBM -> LDS
// once per unit. Wave (qt, kp) scores its 32 queries against key blocks kp and
// kp + 4 and keeps both score blocks in registers, so a single softmax pass
// suffices (no second sweep over K). The next block-row's new K block is fetched
// while the current one is scored, and its queries while it is normalised and
// written.
constexpr int kShortKeys = 512;
constexpr int kShortTileRows = 16;  // query rows per pass of a wave's bf16 output tile

// Block c of a unit's K (keys clamped to nk - 1) as 512 threads move it: wave w
// keys 8w .. 8w + 7, one 16-byte chunk per lane and feature half.
template <int D>
__device__ __forceinline__ void kblock_load(u32x4 x[D / 64], const uint16_t* __restrict__ kseq, int nk, int c) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int m = 8 * wave + (lane >> 3), ch = (lane & 7) ^ ((m >> 1) & 7);
  const int key = min(64 * c + m, nk - 1);
#pragma unroll
  for (int f = 0; f < D / 64; ++f) x[f] = ldg16(kseq + (int64_t)key * D + 64 * f + 8 * ch);
}
template <int D>
__device__ __forceinline__ void kblock_store(uint8_t* kres, int c, const u32x4 x[D / 64]) {
#pragma unroll
  for (int f = 0; f < D / 64; ++f)
    *reinterpret_cast<u32x4*>(kres + (c * (D / 64) + f) * kStageBlockBytes + 16 * threadIdx.x) = x[f];
}

// Largest logit of a score block: raw scores times `scl` (> 0; 1 for blocks
// already turned into logits).
__device__ __forceinline__ float block_max(const f32x16 acc[2], float scl) {
  float b4[4] = {acc[0][0], acc[0][1], acc[0][2], acc[0][3]};
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int v = kt ? 0 : 4; v < 16; ++v) b4[v & 3] = fmaxf(b4[v & 3], acc[kt][v]);
  return fmaxf(fmaxf(b4[0], b4[1]), fmaxf(b4[2], b4[3])) * scl;
}
// acc <- 2^(acc * scl - m) in place; returns this lane's sum of them.
__device__ __forceinline__ float block_exp2(f32x16 acc[2], float scl, float m) {
  float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      acc[kt][v] = exp2f_fast(fmaf(acc[kt][v], scl, -m));
      s4[v & 3] += acc[kt][v];
    }
  return (s4[0] + s4[1]) + (s4[2] + s4[3]);
}

template <int D, bool PACKED, bool OUT_BF16>
__global__ __launch_bounds__(512) void k_attn_maps_short(AttnMapsArgs a) {
  constexpr int FHN = D / 64;
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  uint8_t* kres = reinterpret_cast<uint8_t*>(dyn);
  // 16 rows of a wave's output tile and a spare row that the lanes of the other
  // half write to (their values are not read), so that the tile write needs no branch
  __shared__ __attribute__((aligned(16))) uint32_t wtile[OUT_BF16 ? 8 : 1][OUT_BF16 ? (kShortTileRows + 1) * kTileRow : 1];
  __shared__ float sm[4][64], sl[4][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int qt = wave & 1, kp = wave >> 1, half = lane >> 5;
  const int n_seqs = a.vl.n_seqs, n_units = n_seqs * a.n_heads, stride = gridDim.x;

  // block-rows of unit u; a unit with more keys than the resident K holds is
  // not computed (the lengths must not exceed the maxima the caller passes)
  auto rows_of = [&](int u) {
    const int sq = u % n_seqs;
    const int32_t nq = seq_len_q(a.vl, sq), nk = seq_len_k(a.vl, sq);
    return seq_ok(a.vl, sq, nq, nk) && nq > 0 && nk <= kShortKeys ? (nq + 63) >> 6 : 0;
  };
  // (u, r) -> the workgroup's next item; u = n_units when none is left
  auto advance = [&](int& u, int& r) {
    if (r + 1 < rows_of(u)) {
      ++r;
      return;
    }
    r = 0;
    for (u += stride; u < n_units && rows_of(u) == 0; u += stride) {
    }
  };
  // last key block seen by block-row r
  auto cmax_of = [](int r, int nq, int nk) { return (nk - nq + min(64 * r + 63, nq - 1)) >> 6; };

  // Items of this workgroup: j (being computed) at (u0, r0), then (u1, r1) and
  // (u2, r2); u == n_units: none. Item j computes with the queries fetched during
  // item j - 1 and fetches those of item j + 1; it stores the K block of item
  // j + 1 fetched during item j - 1 and fetches that of item j + 2. Two register
  // sets alternate between consecutive items.
  int u0 = blockIdx.x, r0 = 0;
  while (u0 < n_units && rows_of(u0) == 0) u0 += stride;
  if (u0 >= n_units) return;
  int u1 = u0, r1 = r0;
  advance(u1, r1);
  int u2 = u1, r2 = r1;
  if (u2 < n_units) advance(u2, r2);
  auto kseq_of = [&](int u) {
    return a.k + ((int64_t)(u / n_seqs) * a.vl.total_k + cu_k_of(a.vl, u % n_seqs)) * D;
  };
  // first K block that item (un, rn) adds after item (u, r) (both exist)
  auto first_new = [&](int u, int r, int un, int rn) {
    const int sq = u % n_seqs;
    return un == u ? cmax_of(r, seq_len_q(a.vl, sq), seq_len_k(a.vl, sq)) + 1 : 0;
  };
  QOperand<D> qa, qb;
  u32x4 ka[FHN], kb[FHN];
  {
    const int s = u0 % n_seqs, h = u0 / n_seqs;
    const int32_t nq = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
    const uint16_t* kseq = kseq_of(u0);
    const int c_hi = cmax_of(0, nq, nk);
    for (int c = 0; c <= c_hi; ++c) {
      u32x4 x[FHN];
      kblock_load<D>(x, kseq, nk, c);
      kblock_store<D>(kres, c, x);
    }
    const int i = 32 * qt + (lane & 31);
    load_query_rows<D>(qa, a.q + ((int64_t)h * a.vl.total_q + cu_q_of(a.vl, s) + min(i, nq - 1)) * D);
    // item 1's first new block (a valid address in any case: keys clamped)
    const int un = u1 < n_units ? u1 : u0;
    const int sn = un % n_seqs;
    kblock_load<D>(ka, kseq_of(un), seq_len_k(a.vl, sn), u1 < n_units ? first_new(u0, r0, u1, r1) : 0);
    // Stores through a descriptor of zero bytes (they write nothing), as many as
    // an item issues: the compiler sizes the waits at the loop head by the path
    // into it with the fewest vector memory operations after a load, so without
    // them the entry path would make every item wait for the previous item's
    // stores before its first product.
    const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(a.maps, (short)0, 0, kBufferFlags);
#pragma unroll
    for (int t = 0; t < 48; ++t) __builtin_amdgcn_raw_buffer_store_b32(0u, none, kBufferOff + 4u * t, 0, 0);
  }
  barrier_lds();

  // offset of the current unit's sequence in the map layout, recomputed only when
  // the unit changes (a unit's block-rows are consecutive items)
  int off_u = -1;
  int64_t off_seq = 0;

  // one item; returns whether another follows
  auto item = [&](const QOperand<D>& qop, QOperand<D>& qnext, const u32x4* kcur, u32x4* knext) {
    const int u = u0, r = r0;
    const int s = u % n_seqs, h = u / n_seqs;
    const int32_t nq = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
    const int i = 64 * r + 32 * qt + (lane & 31);
    const bool valid = i < nq;  // rows past the end score a copy of the last row; never stored
    const int last = nk - nq + i;
    const int cmax = cmax_of(r, nq, nk);
    const int cmax_t = (nk - nq + min(64 * r + 32 * qt + 31, nq - 1)) >> 6;
    const int cend = PACKED ? cmax : (nk - 1) >> 6;
    const float scale_l2 = ld_const(a.scale + h) * kLog2e;
    const float bias_l2 = a.bias ? ld_const(a.bias + h) * kLog2e : 0.0f;
    const bool raw_ok = scale_l2 > 0.0f;
    const int first_last = nk - nq + 64 * r + 32 * qt;
    auto lean = [&](int c) { return raw_ok && c != 0 && 64 * c + 63 <= first_last; };
    const bool more = u1 < n_units;

    // scores of blocks kp and kp + 4
    f32x16 acc0[2], acc1[2];
    const int c0 = kp, c1 = kp + 4;
    const bool has0 = c0 <= cmax_t, has1 = c1 <= cmax_t;
    acc0[0] = acc0[1] = acc1[0] = acc1[1] = f32x16{};
    if (has0) {
      kstage_mma<D, 0>(acc0, kres + (c0 * FHN) * kStageBlockBytes, qop);
      if constexpr (FHN == 2) kstage_mma<D, 1>(acc0, kres + (c0 * FHN + 1) * kStageBlockBytes, qop);
    }
    if (has1) {
      kstage_mma<D, 0>(acc1, kres + (c1 * FHN) * kStageBlockBytes, qop);
      if constexpr (FHN == 2) kstage_mma<D, 1>(acc1, kres + (c1 * FHN + 1) * kStageBlockBytes, qop);
    }
    // fetch item j + 1's queries and item j + 2's first new K block (dummy
    // but valid addresses when an item does not exist)
    {
      const int un = more ? u1 : u, rn = more ? r1 : r;
      const int sn = un % n_seqs, hn = un / n_seqs;
      const int32_t nqn = seq_len_q(a.vl, sn);
      const int in = 64 * rn + 32 * qt + (lane & 31);
      load_query_rows<D>(qnext, a.q + ((int64_t)hn * a.vl.total_q + cu_q_of(a.vl, sn) + min(in, nqn - 1)) * D);
      const bool more2 = u2 < n_units;
      const int uk = more2 ? u2 : u;
      kblock_load<D>(knext, kseq_of(uk), seq_len_k(a.vl, uk % n_seqs), more2 ? first_new(u1, r1, u2, r2) : 0);
    }

    // softmax statistics of the wave's two blocks: one max over both, then the
    // blocks become 2^(logit - m) in place and l is their sum
    const bool lean0 = lean(c0), lean1 = lean(c1);
    if (has0 && !lean0) logits_inplace(acc0, 64 * c0, valid ? last : -1, scale_l2, bias_l2);
    if (has1 && !lean1) logits_inplace(acc1, 64 * c1, valid ? last : -1, scale_l2, bias_l2);
    float m = -INFINITY;
    if (has0) m = fmaxf(m, block_max(acc0, lean0 ? scale_l2 : 1.0f));
    if (has1) m = fmaxf(m, block_max(acc1, lean1 ? scale_l2 : 1.0f));
    m = pair32_max(m);
    const float ms = m == -INFINITY ? 0.0f : m;  // every logit -inf: the powers are 0
    float l = 0.0f;
    if (has0) l += block_exp2(acc0, lean0 ? scale_l2 : 1.0f, ms);
    if (has1) l += block_exp2(acc1, lean1 ? scale_l2 : 1.0f, ms);
    l = pair32_add(l);
    if (lane < 32) {
      sm[kp][32 * qt + lane] = m;
      sl[kp][32 * qt + lane] = l;
    }
    barrier_lds();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][32 * qt + (lane & 31)]);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sm[w][32 * qt + (lane & 31)];
      if (mw != -INFINITY) L += sl[w][32 * qt + (lane & 31)] * exp2f_fast(mw - M);
    }
    // p = 2^(logit - m) * 2^(m - M) / L
    const float fac = m == -INFINITY ? 0.0f : exp2f_fast(m - M) * __builtin_amdgcn_rcpf(L);
    // every wave is past its reads of the resident K: item j + 1's blocks go in
    if (more) {
      const int sn = u1 % n_seqs;
      const int lo = u1 == u ? cmax + 1 : 0, hi = cmax_of(r1, seq_len_q(a.vl, sn), seq_len_k(a.vl, sn));
      if (hi >= lo) {
        kblock_store<D>(kres, lo, kcur);
        const uint16_t* kseq_n = kseq_of(u1);
        const int32_t nkn = seq_len_k(a.vl, sn);
        for (int c = lo + 1; c <= hi; ++c) {  // a unit whose first block-row sees several blocks
          u32x4 x[FHN];
          kblock_load<D>(x, kseq_n, nkn, c);
          kblock_store<D>(kres, c, x);
        }
      }
    }
    barrier_lds();

    // normalise and write blocks kp and kp + 4 (zeros past the diagonal of a dense row)
    if (u != off_u) {
      off_seq = map_seq_off(a.vl, s, PACKED);
      off_u = u;
    }
    const int64_t base0 = (int64_t)h * a.head_stride + off_seq;
    uint16_t* region = reinterpret_cast<uint16_t*>(a.maps) + base0;  // this (head, sequence) map
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(region, (short)0, (int)(2 * map_elems(nq, nk, PACKED)), kBufferFlags);
    const int pbase = (int)((reinterpret_cast<uintptr_t>(region) >> 1) & 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = kp + 4 * j;
      const bool live = c <= cend;  // the block exists in the row layout
      f32x16* acc = j ? acc1 : acc0;
      if (!OUT_BF16 && !live) continue;
      if (live) {
        const float f = c <= cmax_t ? fac : 0.0f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[kt][v] *= f;
      }
      if constexpr (OUT_BF16) {
        // Through the wave's LDS tile, 16 query rows at a time: lane (query q,
        // half) puts its 4-key groups at tile row q % 16; then each of 2 passes
        // writes 8 rows, 8 lanes per row and 8 entries per lane, of the block's
        // segment [64c, 64c + len). Stores need 4-byte alignment and a packed row
        // may start at any element, so a lane's 8 entries start at j0 = sh + 8 k
        // (sh: the row's 2-byte phase) and are cut from the tile with a byte
        // shift; the leading entry of an odd-phase row and the partial end of a
        // row go out in 2-, 4- and 8-byte pieces. The stores use a descriptor over
        // this (head, sequence) map; lanes with nothing to write use an offset
        // past it. A block past the row layout issues the same stores, all with
        // that offset: every path then has the same count of vector memory
        // operations, so the compiler's wait for the next item's queries does not
        // also wait for this item's stores.
        uint32_t* tw = wtile[wave];
        const int k8 = lane & 7, rr = lane >> 3;
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
          wave_lds_fence();  // the previous half's reads of the tile come first
          {
            const int trw = ((lane & 31) >> 4) == qh ? (lane & 15) : kShortTileRows;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const u32x2 w = {pack2bf(acc[kt][4 * g], acc[kt][4 * g + 1]),
                                 pack2bf(acc[kt][4 * g + 2], acc[kt][4 * g + 3])};
                *reinterpret_cast<u32x2*>(&tw[trw * kTileRow + 16 * kt + 4 * g + 2 * half]) = w;
              }
          }
          wave_lds_fence();  // rows are read by other lanes
#pragma unroll
          for (int p = 0; p < kShortTileRows / 8; ++p) {
            const int qq = 8 * p + rr;  // tile row
            const int iq = 64 * r + 32 * qt + 16 * qh + qq;
            const int e = (int)map_row_off(iq, nq, nk, PACKED) + 64 * c;  // segment start (element)
            const int len = live && iq < nq ? min(64, (PACKED ? nk - nq + iq + 1 : nk) - 64 * c) : 0;
            const int sh = (pbase + e) & 1, j0 = sh + 8 * k8;
            const uint32_t* trow = tw + qq * kTileRow + 4 * k8;
            const u32x4 w4 = *reinterpret_cast<const u32x4*>(trow);
            const uint32_t w5 = trow[4];
            // entries j0 + 2k, j0 + 2k + 1: the tile's dwords shifted down by sh entries
            auto cut = [sh](uint32_t hi, uint32_t lo) { return sh ? (lo >> 16) | (hi << 16) : lo; };
            const uint32_t d0 = cut(w4[1], w4[0]), d1 = cut(w4[2], w4[1]);
            const uint32_t d2 = cut(w4[3], w4[2]), d3 = cut(w5, w4[3]);
            const uint32_t ob = 2u * (uint32_t)(e + j0);
            const int n = len - j0;  // entries of this lane's 8 inside the segment
            const bool part = n > 0 && n < 8;
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{d0, d1, d2, d3}, rs, n >= 8 ? ob : kBufferOff, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{d0, d1}, rs, part && n >= 4 ? ob : kBufferOff, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(n >= 4 ? d2 : d0, rs, part && (n & 2) ? ob + (n >= 4 ? 8u : 0u) : kBufferOff,
                                                  0, 0);
            const uint32_t dt = n >= 6 ? d3 : n >= 4 ? d2 : n >= 2 ? d1 : d0;  // holds entry n - 1 in its low half
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)dt, rs, part && (n & 1) ? ob + 2u * (uint32_t)(n - 1) : kBufferOff,
                                                  0, 0);
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)w4[0], rs, sh && k8 == 0 && len > 0 ? 2u * (uint32_t)e : kBufferOff,
                                                  0, 0);
          }
        }
      } else {
        if (valid) {
          const int wend = PACKED ? last + 1 : nk;
          const int64_t base = base0 + map_row_off(i, nq, nk, PACKED);
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int key0 = 64 * c + 32 * kt + 8 * g + 4 * half;
              const float p[4] = {acc[kt][4 * g], acc[kt][4 * g + 1], acc[kt][4 * g + 2], acc[kt][4 * g + 3]};
              const int cnt = max(0, min(4, wend - key0));
              if (cnt > 0) store4<OUT_BF16>(a.maps, base + key0, p, cnt);
            }
        }
      }
    }
    u0 = u1;
    r0 = r1;
    u1 = u2;
    r1 = r2;
    if (u2 < n_units) advance(u2, r2);
    return more;
  };
  while (item(qa, qb, ka, kb) && item(qb, qa, kb, ka)) {
  }
}

// Single query rows (decode: one new token per sequence), bf16 inputs. One
// workgroup of 1024 threads per (sequence, head); the dot products are a GEMV, so
// they run on VALU: D/8 lanes share one key row (one 16-byte load each, a wave
// reads whole key rows), reduce across those lanes, and the logit goes to LDS.
// Four keys per group are in flight at a time (256 key rows per workgroup). Max,
// sum and the normalised row are then formed from LDS and written with coalesced
// stores. K is read once when the row fits the LDS window (rows_cap keys, sized
// from the longest key sequence); a longer row (lengths above the maxima the
// caller passed) is still computed, window by window: an online max and sum
// over all windows, then each window's logits again for the write.
constexpr int kRowsThreads = 1024;
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kRowsThreads) void k_attn_rows(AttnMapsArgs a) {
  extern __shared__ float lg[];  // logits (log2 units) of the current window's keys
  constexpr int NW = kRowsThreads / 64;
  __shared__ float red[NW];
  constexpr int LPK = D / 8, KPP = kRowsThreads / LPK;  // lanes per key, keys per pass
  const int s = blockIdx.x, h = blockIdx.y;
  const int32_t nq = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
  if (!seq_ok(a.vl, s, nq, nk) || nq != 1) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l = tid % LPK, g = tid / LPK;
  const uint16_t* qrow = a.q + ((int64_t)h * a.vl.total_q + cu_q_of(a.vl, s)) * D;
  const uint16_t* kseq = a.k + ((int64_t)h * a.vl.total_k + cu_k_of(a.vl, s)) * D;
  const float scale_l2 = ld_const(a.scale + h) * kLog2e;
  const float bias_l2 = a.bias ? ld_const(a.bias + h) * kLog2e : 0.0f;
  const int cap = a.rows_cap;
  float qv[8];
  {
    const u32x4 w = ldg16(qrow + 8 * l);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = __uint_as_float(w[e] << 16);
      qv[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  auto dot = [&](const u32x4& w) {
    float d = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      d = fmaf(qv[2 * e], __uint_as_float(w[e] << 16), d);
      d = fmaf(qv[2 * e + 1], __uint_as_float(w[e] & 0xffff0000u), d);
    }
#pragma unroll
    for (int off = 1; off < LPK; off <<= 1) d += __shfl_xor(d, off, 64);
    return d;
  };
  // logits of keys w0 .. w0 + wn - 1 into lg[0 .. wn); returns this thread's max
  auto logits = [&](int w0, int wn) {
    float mx = -INFINITY;
    int j = g;
    for (; j + 3 * KPP < wn; j += 4 * KPP) {
      u32x4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = ldg16(kseq + (int64_t)(w0 + j + u * KPP) * D + 8 * l);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int key = w0 + j + u * KPP;
        const float t = dot(w[u]) * scale_l2 + (key == 0 ? bias_l2 : 0.0f);
        mx = fmaxf(mx, t);
        if (l == 0) lg[j + u * KPP] = t;
      }
    }
    for (; j < wn; j += KPP) {
      const float t = dot(ldg16(kseq + (int64_t)(w0 + j) * D + 8 * l)) * scale_l2 + (w0 + j == 0 ? bias_l2 : 0.0f);
      mx = fmaxf(mx, t);
      if (l == 0) lg[j] = t;
    }
    return mx;
  };
  // workgroup reductions in a fixed order (the leading barrier also orders the
  // previous use of red and of lg)
  auto wg_max = [&](float x) {
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    __syncthreads();
    if (lane == 0) red[wave] = x;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) m = fmaxf(m, red[w]);
    return m;
  };
  auto wg_sum = [&](float x) {
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    __syncthreads();
    if (lane == 0) red[wave] = x;
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += red[w];
    return t;
  };
  // online max / sum over the windows (one window when nk <= cap)
  float M = -INFINITY, L = 0.0f;
  for (int w0 = 0; w0 < nk; w0 += cap) {
    const int wn = min(cap, nk - w0);
    const float wm = wg_max(logits(w0, wn));
    const float Mn = fmaxf(M, wm);
    float part = 0.0f;
    for (int x = tid; x < wn; x += kRowsThreads) part += exp2f_fast(lg[x] - Mn);
    L = L * exp2f_fast(M - Mn) + wg_sum(part);
    M = Mn;
  }
  const float lse = M + log2f_fast(L);
  const int64_t base = (int64_t)h * a.head_stride + map_seq_off(a.vl, s, a.packed);
  for (int w0 = 0; w0 < nk; w0 += cap) {
    const int wn = min(cap, nk - w0);
    if (nk > cap) {  // the window's logits again (lg holds the last window's)
      __syncthreads();
      logits(w0, wn);
      __syncthreads();
    }
    for (int x = tid; x < wn; x += kRowsThreads) {
      const float p = exp2f_fast(lg[x] - lse);
      if (OUT_BF16) reinterpret_cast<uint16_t*>(a.maps)[base + w0 + x] = f2bf(p);
      else reinterpret_cast<float*>(a.maps)[base + w0 + x] = p;
    }
  }
}

// fp32 inputs: one workgroup per (query row, sequence, head), scores on VALU.
// Used for small fp32 problems; three passes over the keys (max, sum, write).
template <bool PACKED>
__global__ __launch_bounds__(256) void k_attn_maps_f32(AttnMapsArgs a, int d) {
  const int h = blockIdx.z, s = blockIdx.y, i = blockIdx.x;
  const int32_t nq = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
  if (!seq_ok(a.vl, s, nq, nk) || i >= nq) return;
  const float* qrow = a.qf + ((int64_t)h * a.vl.total_q + cu_q_of(a.vl, s) + i) * d;
  const float* kseq = a.kf + ((int64_t)h * a.vl.total_k + cu_k_of(a.vl, s)) * d;
  const float scale = ld_const(a.scale + h), bias = a.bias ? ld_const(a.bias + h) : 0.0f;
  const int last = nk - nq + i;
  __shared__ float red[256];
  auto logit = [&](int j) {
    const float* kr = kseq + (int64_t)j * d;
    float acc = 0.0f;
    for (int e = 0; e < d; ++e) acc = fmaf(qrow[e], kr[e], acc);
    return acc * scale + (j == 0 ? bias : 0.0f);
  };
  float mx = -INFINITY;
  for (int j = threadIdx.x; j <= last; j += 256) mx = fmaxf(mx, logit(j));
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  float sum = 0.0f;
  for (int j = threadIdx.x; j <= last; j += 256) sum += expf(logit(j) - mx);
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const float inv = 1.0f / red[0];
  const int64_t base0 = (int64_t)h * a.head_stride + map_seq_off(a.vl, s, PACKED);
  const int64_t base = base0 + map_row_off(i, nq, nk, PACKED);
  const int wend = PACKED ? last + 1 : nk;
  for (int j = threadIdx.x; j < wend; j += 256) {
    const float p = j <= last ? expf(logit(j) - mx) * inv : 0.0f;
    if (a.out_bf16)
      reinterpret_cast<uint16_t*>(a.maps)[base + j] = f2bf(p);
    else
      reinterpret_cast<float*>(a.maps)[base + j] = p;
  }
}

template <int D, bool PACKED, bool OUT_BF16>
static hipError_t maps_launch(const AttnMapsArgs& a, dim3 grid, hipStream_t st) {
  const size_t lds = 2 * (size_t)kStageBytes;  // the two K stages
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_maps<D, PACKED, OUT_BF16>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  KernelTimer kt_("k_attn_maps", st);
  hipLaunchKernelGGL((k_attn_maps<D, PACKED, OUT_BF16>), grid, dim3(512), lds, st, a);
  return hipGetLastError();
}

// Compute units of the current device (one persistent workgroup each).
int cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int D, bool PACKED, bool OUT_BF16>
static hipError_t short_launch(const AttnMapsArgs& a, int n_wg, hipStream_t st) {
  const size_t lds = (size_t)8 * (D / 64) * kStageBlockBytes;  // the resident K
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_maps_short<D, PACKED, OUT_BF16>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  KernelTimer kt_("k_attn_maps_short", st);
  hipLaunchKernelGGL((k_attn_maps_short<D, PACKED, OUT_BF16>), dim3(n_wg), dim3(512), lds, st, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_short(const AttnMapsArgs& a, hipStream_t st) {
  const int64_t units = (int64_t)a.vl.n_seqs * a.n_heads;
  if (units > INT32_MAX) return hipErrorInvalidValue;
  const int n_wg = (int)std::min<int64_t>(units, cu_count());
  if (a.packed) return a.out_bf16 ? short_launch<D, true, true>(a, n_wg, st) : short_launch<D, true, false>(a, n_wg, st);
  return a.out_bf16 ? short_launch<D, false, true>(a, n_wg, st) : short_launch<D, false, false>(a, n_wg, st);
}

template <int D>
static hipError_t launch_bf16(AttnMapsArgs a, int max_q, hipStream_t st) {
  a.n_rb = (max_q + 63) / 64;
  const int64_t units = (int64_t)a.vl.n_seqs * a.n_heads;
  const int64_t n_wg = 8 * ((units + 7) / 8) * a.n_rb;
  if (n_wg > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n_wg);
  if (a.packed) return a.out_bf16 ? maps_launch<D, true, true>(a, grid, st) : maps_launch<D, true, false>(a, grid, st);
  return a.out_bf16 ? maps_launch<D, false, true>(a, grid, st) : maps_launch<D, false, false>(a, grid, st);
}

constexpr int kRowsMaxKeys = 36 * 1024;  // keys of a single-row sequence held in LDS

template <int D>
static hipError_t launch_rows(AttnMapsArgs a, int max_k, hipStream_t st) {
  a.rows_cap = max_k;  // >= 1 (checked by the caller of launch_rows)
  const size_t lds = (size_t)max_k * sizeof(float);
  const void* f = a.out_bf16 ? reinterpret_cast<const void*>(&k_attn_rows<D, true>)
                             : reinterpret_cast<const void*>(&k_attn_rows<D, false>);
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid(a.vl.n_seqs, a.n_heads);
  if (a.out_bf16) { KernelTimer kt_("k_attn_rows", st); hipLaunchKernelGGL((k_attn_rows<D, true>), grid, dim3(kRowsThreads), lds, st, a); }
  else { KernelTimer kt_("k_attn_rows", st); hipLaunchKernelGGL((k_attn_rows<D, false>), grid, dim3(kRowsThreads), lds, st, a); }
  return hipGetLastError();
}

hipError_t launch_attn_maps(const AttnMapsArgs& a, int d, int max_q, int max_k, hipStream_t st) {
  if (a.n_heads == 0 || a.vl.n_seqs == 0 || max_q == 0) return hipSuccess;
  if (a.in_bf16 && max_q == 1 && max_k >= 1 && max_k <= kRowsMaxKeys) {
    // every sequence has at most one query row (decode)
    return d == 64 ? launch_rows<64>(a, max_k, st) : launch_rows<128>(a, max_k, st);
  }
  if (a.in_bf16 && max_k <= kShortKeys) return d == 64 ? launch_short<64>(a, st) : launch_short<128>(a, st);
  if (a.in_bf16) {
    return d == 64 ? launch_bf16<64>(a, max_q, st) : launch_bf16<128>(a, max_q, st);
  }
  dim3 grid(max_q, a.vl.n_seqs, a.n_heads);
  if (a.packed) { KernelTimer kt_("k_attn_maps_f32", st); hipLaunchKernelGGL((k_attn_maps_f32<true>), grid, dim3(256), 0, st, a, d); }
  else { KernelTimer kt_("k_attn_maps_f32", st); hipLaunchKernelGGL((k_attn_maps_f32<false>), grid, dim3(256), 0, st, a, d); }
  return hipGetLastError();
}

}  // namespace cma
