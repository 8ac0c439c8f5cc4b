// Causal attention probability maps (GLIDE II-B; materialised as IAM Method 4
// requires). Two sweeps per 64-query block-row: the first finds each query's
// softmax max and normaliser with an online update, the second recomputes the
// scores and writes exp(s - max) / sum. Recomputing QK^T is cheaper than a
// round trip of the map: writing the map is the HBM cost of this stage.
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

// grid (n_block_rows, n_seqs, n_heads), 512 threads = 8 waves: wave w owns
// queries 32 (w & 1) .. + 31 of the block-row and key blocks 4k + (w >> 1) of
// each round of the staged K (kstage_pipeline: 4 key blocks x one feature half
// per sub-step, the loads of the sub-step after next in flight). Dynamic LDS:
// the two K stages.
constexpr int kTileRow = 36;  // dwords per row of a wave's bf16 output tile (64 keys + pad)

template <int D, bool PACKED, bool OUT_BF16>
__global__ __launch_bounds__(512) void k_attn_maps(AttnMapsArgs a) {
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  uint8_t* stage = reinterpret_cast<uint8_t*>(dyn);
  __shared__ uint32_t wtile[OUT_BF16 ? 8 : 1][OUT_BF16 ? 32 * kTileRow : 1];
  const int h = blockIdx.z, s = blockIdx.y;
  const int r = (int)gridDim.x - 1 - (int)blockIdx.x;  // longest block-rows first
  const int32_t nq = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
  if (!seq_ok(a.vl, s, nq, nk) || 64 * r >= nq) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int qt = wave & 1, kp = wave >> 1;
  const int i = 64 * r + 32 * qt + (lane & 31);
  const bool valid = i < nq;
  const int last = nk - nq + i;  // last visible key of this query
  const int rowmax = min(64 * r + 63, nq - 1);
  const int cmax = (nk - nq + rowmax) >> 6;  // last key block of the block-row
  // last key block of the wave's queries (past it every key is masked for them)
  const int cmax_t = (nk - nq + min(64 * r + 32 * qt + 31, nq - 1)) >> 6;

  const uint16_t* qrow = a.q + ((int64_t)h * a.vl.total_q + a.vl.cu_q[s] + min(i, nq - 1)) * D;
  const uint16_t* kseq = a.k + ((int64_t)h * a.vl.total_k + a.vl.cu_k[s]) * D;
  const float scale_l2 = a.scale[h] * kLog2e;
  const float bias_l2 = a.bias ? a.bias[h] * kLog2e : 0.0f;

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
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 w = {pack2bf(acc[kt][4 * g], acc[kt][4 * g + 1]), pack2bf(acc[kt][4 * g + 2], acc[kt][4 * g + 3])};
          *reinterpret_cast<u32x2*>(&tw[(lane & 31) * kTileRow + 16 * kt + 4 * g + 2 * half]) = w;
        }
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

// Single query rows (decode: one new token per sequence), bf16 inputs. One
// workgroup of 1024 threads per (sequence, head); the dot products are a GEMV, so
// they run on VALU: D/8 lanes share one key row (one 16-byte load each, a wave
// reads whole key rows), reduce across those lanes, and the logit goes to LDS.
// Four keys per group are in flight at a time (256 key rows per workgroup). Max,
// sum and the normalised row are then formed from LDS and written with coalesced
// stores. K is read once.
constexpr int kRowsThreads = 1024;
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kRowsThreads) void k_attn_rows(AttnMapsArgs a) {
  extern __shared__ float lg[];  // logits (log2 units) of the row's keys
  constexpr int NW = kRowsThreads / 64;
  __shared__ float red[NW];
  constexpr int LPK = D / 8, KPP = kRowsThreads / LPK;  // lanes per key, keys per pass
  const int s = blockIdx.x, h = blockIdx.y;
  const int32_t nq = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
  // rows longer than the LDS sized from max_seqlen_k are not computed (the
  // lengths must not exceed the maxima the caller passes)
  if (!seq_ok(a.vl, s, nq, nk) || nq != 1 || nk > a.rows_cap) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l = tid % LPK, g = tid / LPK;
  const uint16_t* qrow = a.q + ((int64_t)h * a.vl.total_q + a.vl.cu_q[s]) * D;
  const uint16_t* kseq = a.k + ((int64_t)h * a.vl.total_k + a.vl.cu_k[s]) * D;
  const float scale_l2 = a.scale[h] * kLog2e;
  const float bias_l2 = a.bias ? a.bias[h] * kLog2e : 0.0f;
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
  float mx = -INFINITY;
  int j = g;
  for (; j + 3 * KPP < nk; j += 4 * KPP) {
    u32x4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = ldg16(kseq + (int64_t)(j + u * KPP) * D + 8 * l);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = j + u * KPP;
      const float t = dot(w[u]) * scale_l2 + (key == 0 ? bias_l2 : 0.0f);
      mx = fmaxf(mx, t);
      if (l == 0) lg[key] = t;
    }
  }
  for (; j < nk; j += KPP) {
    const float t = dot(ldg16(kseq + (int64_t)j * D + 8 * l)) * scale_l2 + (j == 0 ? bias_l2 : 0.0f);
    mx = fmaxf(mx, t);
    if (l == 0) lg[j] = t;
  }
  // workgroup max, then sum of 2^(t - max), in a fixed order
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, red[w]);
  float sum = 0.0f;
  for (int x = tid; x < nk; x += kRowsThreads) sum += exp2f_fast(lg[x] - M);
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  __syncthreads();
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) L += red[w];
  const float lse = M + log2f_fast(L);
  const int64_t base = (int64_t)h * a.head_stride + map_seq_off(a.vl, s, a.packed);
  for (int x = tid; x < nk; x += kRowsThreads) {
    const float p = exp2f_fast(lg[x] - lse);
    if (OUT_BF16) reinterpret_cast<uint16_t*>(a.maps)[base + x] = f2bf(p);
    else reinterpret_cast<float*>(a.maps)[base + x] = p;
  }
}

// fp32 inputs: one workgroup per (query row, sequence, head), scores on VALU.
// Used for small fp32 problems; three passes over the keys (max, sum, write).
template <bool PACKED>
__global__ __launch_bounds__(256) void k_attn_maps_f32(AttnMapsArgs a, int d) {
  const int h = blockIdx.z, s = blockIdx.y, i = blockIdx.x;
  const int32_t nq = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
  if (!seq_ok(a.vl, s, nq, nk) || i >= nq) return;
  const float* qrow = a.qf + ((int64_t)h * a.vl.total_q + a.vl.cu_q[s] + i) * d;
  const float* kseq = a.kf + ((int64_t)h * a.vl.total_k + a.vl.cu_k[s]) * d;
  const float scale = a.scale[h], bias = a.bias ? a.bias[h] : 0.0f;
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
static void maps_launch(const AttnMapsArgs& a, dim3 grid, hipStream_t st) {
  const size_t lds = 2 * (size_t)kStageBytes;  // the two K stages
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_maps<D, PACKED, OUT_BF16>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  KernelTimer kt_("k_attn_maps", st);
  hipLaunchKernelGGL((k_attn_maps<D, PACKED, OUT_BF16>), grid, dim3(512), lds, st, a);
}

template <int D>
static hipError_t launch_bf16(const AttnMapsArgs& a, dim3 grid, hipStream_t st) {
  if (a.packed) {
    if (a.out_bf16) maps_launch<D, true, true>(a, grid, st);
    else maps_launch<D, true, false>(a, grid, st);
  } else {
    if (a.out_bf16) maps_launch<D, false, true>(a, grid, st);
    else maps_launch<D, false, false>(a, grid, st);
  }
  return hipGetLastError();
}

constexpr int kRowsMaxKeys = 36 * 1024;  // keys of a single-row sequence held in LDS

template <int D>
static hipError_t launch_rows(AttnMapsArgs a, int max_k, hipStream_t st) {
  a.rows_cap = max_k;
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
  if (a.in_bf16) {
    dim3 grid((max_q + 63) / 64, a.vl.n_seqs, a.n_heads);
    return d == 64 ? launch_bf16<64>(a, grid, st) : launch_bf16<128>(a, grid, st);
  }
  dim3 grid(max_q, a.vl.n_seqs, a.n_heads);
  if (a.packed) { KernelTimer kt_("k_attn_maps_f32", st); hipLaunchKernelGGL((k_attn_maps_f32<true>), grid, dim3(256), 0, st, a, d); }
  else { KernelTimer kt_("k_attn_maps_f32", st); hipLaunchKernelGGL((k_attn_maps_f32<false>), grid, dim3(256), 0, st, a, d); }
  return hipGetLastError();
}

}  // namespace cma
