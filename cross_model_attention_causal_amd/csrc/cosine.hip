// Head mapping by cosine similarity of flattened maps (IAM Methods 1 and 4).
//
// The cosine matrix is a Gram product R S^T over the map length with the row
// norms on the side. It runs as a split-K bf16 MFMA GEMM (32x32x16): a
// workgroup (8 waves) owns 128 receiver maps and one K-chunk and holds the
// partial dot products of its 128 maps against all sender maps in registers
// (wave = 32 receivers x one half of the 32-sender tiles). Each 64-element K-step
// of the tile's receiver maps and of the sender maps is staged in LDS (each map
// read once per workgroup) by a depth-2 pipeline: while a step's products run,
// the loads of the step after next are in flight into registers and the next
// step goes to the other LDS buffer. Partial sums of each split go to a
// workspace and a finalize kernel adds them in a fixed order (deterministic),
// forms the cosines and takes argmax (lowest index on ties) and margin.
#include "kernels.hpp"
#include "score.hpp"

namespace cma {

constexpr int kGramRows = 128;     // receiver maps per workgroup
constexpr int kGramK = 64;         // K elements per step
constexpr int kGramThreads = 512;  // 8 waves = 4 groups of 32 receivers x 2 halves of the sender tiles
constexpr int kMaxSteps = 128;     // K-steps of one split (8192 elements)

// The sender slice of a step in LDS: row j (a sender map) holds 64 elements as 8
// chunks of 16 bytes, chunk ch in slot ch ^ ((j >> 1) & 7), so that the 16 rows
// one operand read touches fall in distinct bank groups.
__device__ __forceinline__ int sslot(int row, int ch) { return row * 8 + (ch ^ ((row >> 1) & 7)); }

// t + lo^2 + hi^2 for the two bf16 values packed in w (one dot2 instruction; the
// products of bf16 values are exact in fp32)
__device__ __forceinline__ float sq2(uint32_t w, float t) {
  const bf16x2 x = __builtin_bit_cast(bf16x2, w);
  return __builtin_amdgcn_fdot2_f32_bf16(x, x, t, false);
}

// NTH: staged sender tiles of 32 (n_send <= 32 * NTH); DEPTH: steps whose loads
// are in flight while a step is computed (2 needs a second register set).
template <int NTH, int DEPTH>
__global__ __launch_bounds__(kGramThreads) void k_gram_bf16(CosineArgs a) {
  constexpr int SROWS = 32 * NTH;                                  // staged sender rows
  constexpr int T2 = (NTH + 1) / 2;                                // sender tiles per wave
  constexpr int ROWS = kGramRows + SROWS;                          // staged rows: receivers, then senders
  constexpr int CH = ROWS * 8;                                     // 16-byte chunks per stage
  constexpr int PT = (CH + kGramThreads - 1) / kGramThreads;       // chunks per thread
  __shared__ __attribute__((aligned(16))) u32x4 sb[2][CH];
  const int b = blockIdx.y;
  const int n_rtiles = (a.n_recv + kGramRows - 1) / kGramRows;
  // Workgroup id i runs on XCD i % 8. Split sp goes to XCD sp % 8 with all its
  // receiver tiles in consecutive slots there, so the tiles of a split run
  // together and share its sender slice through that XCD's L2.
  const int xcd = blockIdx.x % kXcds, m = blockIdx.x / kXcds;
  const int sp = xcd + kXcds * (m / n_rtiles), rt = m % n_rtiles;
  if (sp >= a.splits) return;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int nl = lane & 31, hl = lane >> 5;
  const int rg = wave & 3, sh = wave >> 2;  // receiver group, half of the sender tiles
  const int64_t k_beg = (int64_t)sp * a.kchunk;
  const int64_t k_end = min(a.len, k_beg + a.kchunk);
  const int nsteps = (int)((k_end - k_beg + kGramK - 1) / kGramK);
  const uint16_t* recv = reinterpret_cast<const uint16_t*>(a.recv) + (int64_t)b * a.rb;
  const uint16_t* send = reinterpret_cast<const uint16_t*>(a.send) + (int64_t)b * a.sb;
  const int rbase = rt * kGramRows;
  const int row0 = rbase + 32 * rg;

  f32x16 acc[T2];
#pragma unroll
  for (int t = 0; t < T2; ++t) acc[t] = f32x16{};
  // Squared norms in two levels: a step's squares are summed apart, added to an
  // inner running sum that is folded into the outer one every 16 steps. A single
  // long fp32 chain would drop the many tiny squares of a probability map's tail
  // once the sum has grown (a systematic underestimate, which biases the cosine).
  float rn = 0.f, rn_in = 0.f;
  float sn = 0.f, sn_in = 0.f;
  // sender rows whose norms this workgroup accumulates (one per thread): the
  // receiver tiles of a split share the rows out
  const int s_per = (a.n_send + n_rtiles - 1) / n_rtiles;
  const int srow = rt * s_per + tid;
  const bool s_mine = tid < s_per && srow < a.n_send;

  // A step's stage: the 64 elements of the tile's 128 receiver maps, then those
  // of the staged sender maps; staged row j holds 8 chunks of 16 bytes, chunk ch
  // in slot ch ^ ((j >> 1) & 7). Thread chunk i is x = tid + 512 i = (row x / 8,
  // slot x % 8), read from a fixed map row: rows past the last map read a valid
  // row, whose products and norms are never stored. Each map is read once per
  // workgroup and both sender halves take their receiver operands from LDS.
  const uint16_t* cptr[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int x = min(tid + kGramThreads * i, CH - 1), row = x >> 3, slot = x & 7;
    const int ch = slot ^ ((row >> 1) & 7);
    const uint16_t* base = row < kGramRows ? recv + (int64_t)min(rbase + row, a.n_recv - 1) * a.rh
                                           : send + (int64_t)min(row - kGramRows, a.n_send - 1) * a.sh;
    cptr[i] = base + 8 * ch;
  }
  auto load = [&](int st, u32x4 (&v)[PT], auto guarded) __attribute__((always_inline)) {
    const int64_t k0 = k_beg + (int64_t)st * kGramK;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      if constexpr (decltype(guarded)::value) {
        // element-guarded: chunk offset of the row pointer within the 64 elements
        const int x = min(tid + kGramThreads * i, CH - 1), row = x >> 3, slot = x & 7;
        const int ch = slot ^ ((row >> 1) & 7);
        v[i] = ldg16_guard(cptr[i] - 8 * ch, k0 + 8 * ch, k_end);
      } else {
        v[i] = ldg16(cptr[i] + k0);
      }
    }
  };
  auto store = [&](const u32x4 (&v)[PT], int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int x = tid + kGramThreads * i;
      if (CH % kGramThreads == 0 || x < CH) sb[buf][x] = v[i];  // slot order: x = row * 8 + slot
    }
  };
  // one step's work on the stage in LDS buffer buf. Operands of 32x32x16: lane
  // (nl, hl) holds elements 16 ks + 8 hl .. + 7 of map row nl of the tile (A:
  // receivers, B: senders), so that D[m][n] = sum_k R[m][k] S[n][k].
  auto compute = [&](int st, int buf) __attribute__((always_inline)) {
    u32x4 av[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) av[ks] = sb[buf][sslot(32 * rg + nl, 2 * ks + hl)];
    // receiver norms (one sender half does it; the partner lane holds the other
    // half of the row's elements)
    if (sh == 0) {
      float t = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) t = sq2(av[ks][e], t);
      rn_in += t;
    }
    // sender norms of this workgroup's share of the rows, in element order
    if (s_mine) {
      float t = 0.0f;
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        const u32x4 v = sb[buf][sslot(kGramRows + srow, ch)];
#pragma unroll
        for (int e = 0; e < 4; ++e) t = sq2(v[e], t);
      }
      sn_in += t;
    }
    if (((st + 1) & 15) == 0) {
      rn += rn_in;
      rn_in = 0.0f;
      sn += sn_in;
      sn_in = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < T2; ++t) {
      const int tile = sh * T2 + t;
      if (tile < NTH) {
        const int srow_b = kGramRows + 32 * tile + nl;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4 bv = sb[buf][sslot(srow_b, 2 * ks + hl)];
          acc[t] = mfma32(as_bf16x8(av[ks]), as_bf16x8(bv), acc[t]);
        }
      }
    }
  };

  using Fast = std::integral_constant<bool, false>;
  using Guarded = std::integral_constant<bool, true>;
  const int nfull = (int)((k_end - k_beg) / kGramK);  // steps with all 64 elements inside the chunk
  // Pipeline of depth 2: while step st is computed from one LDS buffer, the
  // loads of step st + 2 are in flight into registers and step st + 1 (loaded
  // one iteration earlier) goes to the other buffer. Past the last full step the
  // loads are clamped (harmless reloads) and nothing is computed, so that both
  // register sets see the same operations on every path and the compiler's
  // waits for the older set never include the newer one. Depth 1: the loads of
  // step st + 1 are in flight while step st is computed.
  u32x4 r0[PT];
  if constexpr (DEPTH == 2) {
    u32x4 r1[PT];
    if (nfull > 0) {
      load(0, r0, Fast{});
      load(min(1, nfull - 1), r1, Fast{});
      store(r0, 0);
    }
    __syncthreads();
    auto iter = [&](u32x4 (&mine)[PT], const u32x4 (&next)[PT], int st) __attribute__((always_inline)) {
      load(min(st + 2, nfull - 1), mine, Fast{});
      if (st < nfull) compute(st, st & 1);
      store(next, (st + 1) & 1);
      __syncthreads();
    };
    for (int st = 0; st < nfull; st += 2) {
      iter(r0, r1, st);
      iter(r1, r0, st + 1);
    }
  } else {
    if (nfull > 0) {
      load(0, r0, Fast{});
      store(r0, 0);
    }
    __syncthreads();
    for (int st = 0; st < nfull; ++st) {
      load(min(st + 1, nfull - 1), r0, Fast{});
      compute(st, st & 1);
      store(r0, (st + 1) & 1);
      __syncthreads();
    }
  }
  if (nfull < nsteps) {
    // the partial last step
    load(nfull, r0, Guarded{});
    store(r0, 0);
    __syncthreads();
    compute(nfull, 0);
  }

  rn += rn_in;
  sn += sn_in;
  // partial dot products: D[m = 8 (v / 4) + 4 hl + v % 4][n = nl]
  float* part = a.part + ((int64_t)sp * a.n_batch + b) * a.n_recv * a.n_send;
#pragma unroll
  for (int t = 0; t < T2; ++t) {
    const int col = 32 * (sh * T2 + t) + nl;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = row0 + 8 * (v >> 2) + 4 * hl + (v & 3);
      if (row < a.n_recv && col < a.n_send) part[(int64_t)row * a.n_send + col] = acc[t][v];
    }
  }
  if (sh == 0) {
    const float x = rn + xor_lane(rn, 32);
    const int row = row0 + nl;
    if (hl == 0 && row < a.n_recv) a.rnorm[((int64_t)sp * a.n_batch + b) * a.n_recv + row] = x;
  }
  if (s_mine) a.snorm[((int64_t)sp * a.n_batch + b) * a.n_send + srow] = sn;
}

// fp32 maps: one workgroup per (sender, receiver, problem), VALU dot products.
__global__ __launch_bounds__(256) void k_gram_f32(CosineArgs a) {
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const float* r = reinterpret_cast<const float*>(a.recv) + (int64_t)b * a.rb + (int64_t)h * a.rh;
  const float* s = reinterpret_cast<const float*>(a.send) + (int64_t)b * a.sb + (int64_t)j * a.sh;
  float dot = 0.f, rr = 0.f, ss = 0.f;
  for (int64_t e = threadIdx.x; e < a.len; e += 256) {
    const float x = r[e], y = s[e];
    dot = fmaf(x, y, dot);
    rr = fmaf(x, x, rr);
    ss = fmaf(y, y, ss);
  }
  __shared__ float red[3][256];
  red[0][threadIdx.x] = dot;
  red[1][threadIdx.x] = rr;
  red[2][threadIdx.x] = ss;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w)
      for (int t = 0; t < 3; ++t) red[t][threadIdx.x] += red[t][threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.part[((int64_t)b * a.n_recv + h) * a.n_send + j] = red[0][0];
    if (j == 0) a.rnorm[(int64_t)b * a.n_recv + h] = red[1][0];
    if (h == 0) a.snorm[(int64_t)b * a.n_send + j] = red[2][0];
  }
}

// Better of two (value, index) candidates: larger value, lower index on ties.
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// Top-2 of (value, index) pairs under `better`, a strict total order (ties to
// the lower index): merging partial lists in any order gives the same result.
__device__ __forceinline__ void top2_merge(float& v1, int& i1, float& v2, int& i2, float ov1, int oi1, float ov2,
                                           int oi2) {
  float n1, n2;
  int j1, j2;
  if (better(v1, i1, ov1, oi1)) {
    n1 = v1; j1 = i1;
    if (better(v2, i2, ov1, oi1)) { n2 = v2; j2 = i2; } else { n2 = ov1; j2 = oi1; }
  } else {
    n1 = ov1; j1 = oi1;
    if (better(v1, i1, ov2, oi2)) { n2 = v1; j2 = i1; } else { n2 = ov2; j2 = oi2; }
  }
  v1 = n1; i1 = j1; v2 = n2; i2 = j2;
}

// One workgroup of 256 threads per (receiver map, problem); thread t forms the
// cosines of senders t, t + 256, ... Each cosine adds its splits' partial dot
// products and sender norms in four interleaved sums (split sp into sum sp % 4,
// in increasing sp), eight partials in flight; then the top two cosines per
// wave, merged through LDS.
constexpr int kFinThreads = 256;
__global__ __launch_bounds__(kFinThreads) void k_cos_finalize(CosineArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float sv[2][kFinThreads / 64];
  __shared__ int si[2][kFinThreads / 64];
  // the receiver's norm: its splits' partial sums, added in split order (scalar
  // loads of the Gram's output, issued back to back)
  float rn = 0.f;
#pragma unroll 8
  for (int sp = 0; sp < a.splits; ++sp) rn += ld_const(a.rnorm + ((int64_t)sp * a.n_batch + b) * a.n_recv + h);
  const float rs = sqrtf(rn);
  float v1 = -INFINITY, v2 = -INFINITY;
  int i1 = 0x7fffffff, i2 = 0x7fffffff;
  const int64_t pstride = (int64_t)a.n_batch * a.n_recv * a.n_send, sstride = (int64_t)a.n_batch * a.n_send;
  for (int j = tid; j < a.n_send; j += kFinThreads) {
    float d4[4] = {0.f, 0.f, 0.f, 0.f}, s4[4] = {0.f, 0.f, 0.f, 0.f};
    const float* pp = a.part + ((int64_t)b * a.n_recv + h) * a.n_send + j;
    const float* ps = a.snorm + (int64_t)b * a.n_send + j;
    int sp = 0;
    for (; sp + 7 < a.splits; sp += 8) {
      float pd[8], pn[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        pd[u] = pp[(sp + u) * pstride];
        pn[u] = ps[(sp + u) * sstride];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        d4[u & 3] += pd[u];
        s4[u & 3] += pn[u];
      }
    }
    for (int u = 0; sp < a.splits; ++sp, ++u) {
      d4[u & 3] += pp[sp * pstride];
      s4[u & 3] += ps[sp * sstride];
    }
    const float dot = (d4[0] + d4[1]) + (d4[2] + d4[3]), sn = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    const float den = rs * sqrtf(sn);
    const float c = den > 0.f ? dot / den : 0.f;
    if (a.cos) a.cos[((int64_t)b * a.n_recv + h) * a.n_send + j] = c;
    if (better(c, j, v1, i1)) {
      v2 = v1; i2 = i1; v1 = c; i1 = j;
    } else if (better(c, j, v2, i2)) {
      v2 = c; i2 = j;
    }
  }
  for (int off = 32; off > 0; off >>= 1)
    top2_merge(v1, i1, v2, i2, __shfl_xor(v1, off, 64), __shfl_xor(i1, off, 64), __shfl_xor(v2, off, 64),
               __shfl_xor(i2, off, 64));
  if (lane == 0) {
    sv[0][wave] = v1; si[0][wave] = i1;
    sv[1][wave] = v2; si[1][wave] = i2;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kFinThreads / 64; ++w) top2_merge(v1, i1, v2, i2, sv[0][w], si[0][w], sv[1][w], si[1][w]);
    a.argmax[(int64_t)b * a.n_recv + h] = i1;
    if (a.margin) a.margin[(int64_t)b * a.n_recv + h] = a.n_send > 1 ? v1 - v2 : INFINITY;
  }
}

// ------------------------------------------------------------ fused maps -> cosine
// Head mapping without storing the receivers' maps (IAM Methods 1 and 4: the
// cosine of flattened causal maps; the maps are explicit softmax outputs, so no
// flash-style kernel can produce them): a workgroup owns 32 query rows of one
// sequence (one split of the Gram's K), 32 receiver heads and up to 128 sender
// heads. It first sweeps the keys once per head for the rows' softmax statistics
// (online max and sum, 32x32x16 bf16 MFMA), then walks the rows' keys in blocks
// of 32: the waves recompute their heads' score tiles, form the probabilities,
// round them to bf16 (the values a stored map would hold) and write them to an
// LDS buffer ordered (row, head, key), double-buffered; the same waves then take
// rows of the buffer as the A operand (32 heads x 16 keys) of 32x32x16 MFMAs
// whose B operand is the sender maps' same row and keys (dense bf16 maps, read
// straight into registers). Per split the Gram partial, the receivers' squared
// norms (from the rounded values) and the senders' squared norms go to the
// workspace; k_cos_finalize adds the splits in a fixed order.
constexpr int kFusedRS = kFusedHeads * 64 + 16;   // LDS bytes per query row of a buffer
constexpr int kFusedBuf = kFusedRows * kFusedRS;  // one buffer

__global__ __launch_bounds__(512) void k_head_map_fused(FusedMapArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float lse_s[kFusedHeads][kFusedRows];
  __shared__ float sn_s[24][32];  // senders' squared norms per Gram item
  const int n_rt = (a.n_recv + kFusedHeads - 1) / kFusedHeads, n_sg = (a.n_send + kFusedSend - 1) / kFusedSend;
  const int per_qt = n_rt * n_sg;
  const int qt = a.n_qt - 1 - (int)(blockIdx.x / per_qt);  // the longest splits first
  const int rem = (int)(blockIdx.x % per_qt), sg = rem / n_rt, rt = rem % n_rt;
  const int b = blockIdx.y;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int nl = lane & 31, hl = lane >> 5;
  const int32_t n = seq_len_q(a.vl, b), nk = seq_len_k(a.vl, b);
  const int i0 = kFusedRows * qt;
  const int64_t split_row = (int64_t)qt * a.fin.n_batch + b;
  float* part = a.fin.part + split_row * a.n_recv * a.n_send;
  if (!seq_ok(a.vl, b, n, nk) || n != nk || i0 >= n) {
    // no rows of this problem in this split: its partials are zero
    for (int x = tid; x < kFusedHeads * kFusedSend; x += 512) {
      const int h = kFusedHeads * rt + x / kFusedSend, j = kFusedSend * sg + x % kFusedSend;
      if (h < a.n_recv && j < a.n_send) part[(int64_t)h * a.n_send + j] = 0.f;
    }
    if (sg == 0 && tid < kFusedHeads && kFusedHeads * rt + tid < a.n_recv)
      a.fin.rnorm[split_row * a.n_recv + kFusedHeads * rt + tid] = 0.f;
    if (rt == 0 && tid < kFusedSend && kFusedSend * sg + tid < a.n_send)
      a.fin.snorm[split_row * a.n_send + kFusedSend * sg + tid] = 0.f;
    return;
  }
  const int64_t q0 = cu_q_of(a.vl, b), k0 = cu_k_of(a.vl, b);
  const int64_t map_off = map_seq_off(a.vl, b, false);  // the sequence's dense sender maps
  const int n_kb = qt + 1;                               // key blocks of 32: keys 0 .. i0 + 31
  const int qpos = i0 + nl;                              // the lane's query row
  const bool qvalid = qpos < n;
  const bool do_snorm = rt == 0;

  // this lane's Q operand of head h (B of 32x32x16: query nl, features 16 ks + 8 hl ..)
  auto load_q = [&](int h, QOperand<128>& qop) __attribute__((always_inline)) {
    load_query_clamped<128>(qop, a.q + ((int64_t)h * a.vl.total_q + q0 + min(qpos, n - 1)) * 128, qvalid);
  };
  // the K operand of key block kb (32 keys; A of 32x32x16: key nl, features 16 ks + 8 hl ..)
  auto load_kt = [&](int h, int kb, u32x4 (&kx)[8]) __attribute__((always_inline)) {
    const int key = min(32 * kb + nl, n - 1);
    const uint16_t* krow = a.k + ((int64_t)h * a.vl.total_k + k0 + key) * 128 + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kx[ks] = ldg16(krow + 16 * ks);
  };
  // scores of a key block x the 32 queries: D[key 8(v/4) + 4 hl + v%4][query nl]
  auto mma_kt = [&](const u32x4 (&kx)[8], const QOperand<128>& qop) __attribute__((always_inline)) {
    f32x16 c = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) c = mfma32(as_bf16x8(kx[ks]), qop.v[ks], c);
    return c;
  };
  auto key_of = [&](int kb, int v) __attribute__((always_inline)) { return 32 * kb + 8 * (v >> 2) + 4 * hl + (v & 3); };

  // ---- softmax statistics of the 32 rows, per head (wave w: heads 4w .. 4w + 3)
#pragma unroll 1
  for (int u = 0; u < 4; ++u) {
    const int hh = 4 * wave + u, h = kFusedHeads * rt + hh;
    float lse = -INFINITY;
    if (h < a.n_recv) {
      QOperand<128> qop;
      load_q(h, qop);
      const float sl2 = ld_const(a.scale + h) * kLog2e, bl2 = a.bias ? ld_const(a.bias + h) * kLog2e : 0.0f;
      float m = -INFINITY, l = 0.0f;
      // key blocks two at a time, the next block's K in flight during a block's products
      u32x4 kxa[8], kxb[8];
      load_kt(h, 0, kxa);
      auto step = [&](int kb, const u32x4 (&kx)[8]) __attribute__((always_inline)) {
        f32x16 c = mma_kt(kx, qop);
        float bm = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = key_of(kb, v);
          const float t = (key <= qpos && key < n) ? c[v] * sl2 + (key == 0 ? bl2 : 0.0f) : -INFINITY;
          c[v] = t;
          bm = fmaxf(bm, t);
        }
        bm = pair32_max(bm);
        const float mn = fmaxf(m, bm);
        float s = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) s += mn == -INFINITY ? 0.0f : exp2f_fast(c[v] - mn);
        s = pair32_add(s);
        l = mn == -INFINITY ? 0.0f : l * exp2f_fast(m - mn) + s;
        m = mn;
      };
      for (int kb = 0; kb < n_kb; kb += 2) {
        if (kb + 1 < n_kb) load_kt(h, kb + 1, kxb);
        step(kb, kxa);
        if (kb + 1 < n_kb) {
          if (kb + 2 < n_kb) load_kt(h, kb + 2, kxa);
          step(kb + 1, kxb);
        }
      }
      lse = m + log2f_fast(l);
    }
    if (lane < 32) lse_s[hh][lane] = lse;
  }
  __syncthreads();

  // ---- probabilities into the LDS buffer, then the Gram
  // The Gram of a key block is split into items (32-sender tile t, group g of
  // 32 / G rows), dealt round robin to the waves (at most 3 per wave): G rows
  // groups per tile so that there are at least 8 items however few senders.
  const int n_tiles = (min(kFusedSend, a.n_send - kFusedSend * sg) + 31) / 32;
  const int G = n_tiles >= 6 ? 2 : (n_tiles >= 3 ? 4 : 8), RG = kFusedRows / G;
  const int n_items = n_tiles * G;
  f32x16 acc[3];
#pragma unroll
  for (int it = 0; it < 3; ++it) acc[it] = f32x16{};
  float rn[4] = {0.f, 0.f, 0.f, 0.f}, sn[3] = {0.f, 0.f, 0.f};
  // Produce key block kb into buffer buf: lane (query nl, half hl) writes its 16
  // probabilities of each head as four 8-byte pieces at row nl, head slot hh,
  // 8-key chunk g placed at slot g ^ ((hh >> 1) & 3) (the reads of 32 heads then
  // spread over the bank groups); the row stride's extra 16 bytes spread the 32
  // rows a write touches.
  auto produce = [&](int kb, int buf) __attribute__((always_inline)) {
    uint8_t* B = smem + buf * kFusedBuf;
#pragma unroll 1
    for (int u = 0; u < 4; ++u) {
      const int hh = 4 * wave + u, h = kFusedHeads * rt + hh;
      uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
      if (h < a.n_recv) {
        QOperand<128> qop;
        u32x4 kx[8];
        load_q(h, qop);
        load_kt(h, kb, kx);
        const f32x16 c = mma_kt(kx, qop);
        const float sl2 = ld_const(a.scale + h) * kLog2e, bl2 = a.bias ? ld_const(a.bias + h) * kLog2e : 0.0f;
        const float lse = lse_s[hh][nl];
        float p[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = key_of(kb, v);
          const float t = c[v] * sl2 + (key == 0 ? bl2 : 0.0f);
          p[v] = (qvalid && key <= qpos) ? exp2f_fast(t - lse) : 0.0f;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          w[2 * g] = pack2bf(p[4 * g], p[4 * g + 1]);
          w[2 * g + 1] = pack2bf(p[4 * g + 2], p[4 * g + 3]);
        }
        float t = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) t = sq2(w[e], t);
        rn[u] += t;  // one tile's squares at a time (a short chain per lane)
      }
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<u32x2*>(B + nl * kFusedRS + hh * 64 + 16 * (g ^ ((hh >> 1) & 3)) + 8 * hl) =
            u32x2{w[2 * g], w[2 * g + 1]};
    }
  };
  // sender operands (B of 32x32x16: sender 32 t + nl, keys key0 + 8 hl ..) of row
  // i: FAST (every row starts on 16 bytes and the sequence fills whole key blocks)
  // takes plain 16-byte loads with no branch, else each load checks alignment and
  // the row's end
  auto load_b = [&](int t, int i, int kb, u32x4 (&bv)[2], auto fast) __attribute__((always_inline)) {
    const int jr = kFusedSend * sg + 32 * t + nl;
    const int64_t so = (int64_t)min(jr, a.n_send - 1) * a.send_hs + map_off + (int64_t)min(i, n - 1) * n;
    const uint16_t* srow = a.send + so;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int key0 = 32 * kb + 16 * ks + 8 * hl;
      if constexpr (decltype(fast)::value) {
        bv[ks] = ldg16(srow + key0);
      } else {
        bv[ks] = (((so + key0) & 7) == 0 && key0 + 8 <= n) ? ldg16(srow + key0) : ldg16_guard_any(srow, key0, n);
      }
    }
  };
  const bool fast = (n % 32) == 0 && (map_off % 8) == 0 && (a.send_hs % 8) == 0 &&
                    (reinterpret_cast<uintptr_t>(a.send) & 15) == 0;
  // Gram of key block kb from buffer buf: this wave's items, rows two at a time
  // with the sender operands of the next two rows in flight (rows past the
  // sequence end read the last row; their probabilities in the buffer are zero)
  auto consume = [&](int kb, int buf, auto fastc) __attribute__((always_inline)) {
    const uint8_t* B = smem + buf * kFusedBuf;
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const int item = wave + 8 * it;
      if (item >= n_items) break;
      const int t = item / G, r0 = (item % G) * RG;
      if (i0 + r0 >= n) continue;
      u32x4 bc[2][2], bn[2][2];
#pragma unroll
      for (int e = 0; e < 2; ++e) load_b(t, i0 + r0 + e, kb, bc[e], fastc);
      for (int r = r0; r < r0 + RG; r += 2) {
        if (r + 2 < r0 + RG) {
#pragma unroll
          for (int e = 0; e < 2; ++e) load_b(t, i0 + r + 2 + e, kb, bn[e], fastc);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int c8 = 2 * ks + hl;
            const u32x4 av =
                *reinterpret_cast<const u32x4*>(B + (r + e) * kFusedRS + nl * 64 + 16 * (c8 ^ ((nl >> 1) & 3)));
            acc[it] = mfma32(as_bf16x8(av), as_bf16x8(bc[e][ks]), acc[it]);
            if (do_snorm && i0 + r + e < n) {
              float q2 = 0.0f;
#pragma unroll
              for (int x = 0; x < 4; ++x) q2 = sq2(bc[e][ks][x], q2);
              sn[it] += q2;
            }
          }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          bc[e][0] = bn[e][0];
          bc[e][1] = bn[e][1];
        }
      }
    }
  };
  produce(0, 0);
  __syncthreads();
  for (int kb = 0; kb < n_kb; ++kb) {
    if (kb + 1 < n_kb) produce(kb + 1, (kb + 1) & 1);
    if (fast) consume(kb, kb & 1, std::true_type{});
    else consume(kb, kb & 1, std::false_type{});
    __syncthreads();
  }

  // ---- partial Gram: per tile, the row groups' sums added in group order
  float* red = reinterpret_cast<float*>(smem);  // [item][32 heads][32 senders]
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    const int item = wave + 8 * it;
    if (item < n_items) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = 8 * (v >> 2) + 4 * hl + (v & 3);
        red[(item * kFusedHeads + m) * 32 + nl] = acc[it][v];
      }
      if (do_snorm) {
        const float x = pair32_add(sn[it]);
        if (lane < 32) sn_s[item][nl] = x;
      }
    }
  }
  // receivers' squared norms: wave w's heads, over its lanes
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float x = rn[u];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x += xor_lane(x, off);
    const int h = kFusedHeads * rt + 4 * wave + u;
    if (sg == 0 && lane == 0 && h < a.n_recv) a.fin.rnorm[split_row * a.n_recv + h] = x;
  }
  __syncthreads();
  for (int x = tid; x < kFusedHeads * 32 * n_tiles; x += 512) {
    const int t = x / (kFusedHeads * 32), y = x % (kFusedHeads * 32), m = y / 32, jj = y % 32;
    float s = 0.0f;
    for (int g = 0; g < G; ++g) s += red[((t * G + g) * kFusedHeads + m) * 32 + jj];
    const int h = kFusedHeads * rt + m, j = kFusedSend * sg + 32 * t + jj;
    if (h < a.n_recv && j < a.n_send) part[(int64_t)h * a.n_send + j] = s;
  }
  if (do_snorm && tid < 32 * n_tiles && kFusedSend * sg + tid < a.n_send) {
    const int t = tid / 32, jj = tid % 32;
    float s = 0.0f;
    for (int g = 0; g < G; ++g) s += sn_s[t * G + g][jj];
    a.fin.snorm[split_row * a.n_send + kFusedSend * sg + tid] = s;
  }
}

size_t fused_map_ws_bytes(int32_t n_batch, int32_t n_recv, int32_t n_send, int32_t max_seqlen) {
  const int64_t n_qt = (max_seqlen + kFusedRows - 1) / kFusedRows;
  return (size_t)n_qt * n_batch * ((size_t)n_recv * n_send + n_recv + n_send) * sizeof(float);
}

hipError_t launch_head_map_fused(const FusedMapArgs& a, hipStream_t st) {
  if (a.fin.n_batch == 0 || a.n_recv == 0 || a.n_qt == 0) return hipSuccess;
  const int n_rt = (a.n_recv + kFusedHeads - 1) / kFusedHeads, n_sg = (a.n_send + kFusedSend - 1) / kFusedSend;
  const size_t lds = 2 * (size_t)kFusedBuf;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_head_map_fused),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  {
    KernelTimer kt_("k_head_map_fused", st);
    hipLaunchKernelGGL(k_head_map_fused, dim3((unsigned)(a.n_qt * n_rt * n_sg), a.fin.n_batch), dim3(512), lds, st,
                       a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  { KernelTimer kt_("k_cos_finalize", st); hipLaunchKernelGGL(k_cos_finalize, dim3(a.n_recv, a.fin.n_batch), dim3(kFinThreads), 0, st, a.fin); }
  return hipGetLastError();
}

CosinePlan plan_cosine(int32_t n_batch, int32_t n_recv, int32_t n_send, int64_t len, bool bf16) {
  CosinePlan pl;
  if (!bf16) {
    pl.splits = 1;
    pl.kchunk = len;
  } else {
    const int64_t kblocks = (len + kGramK - 1) / kGramK;
    const int64_t tiles = (int64_t)((n_recv + kGramRows - 1) / kGramRows) * n_batch;
    // At most kMaxSteps K-steps per split, so that each partial dot product is a
    // short fp32 accumulation chain, and at least one workgroup per CU (one fits
    // at a time); among the step counts that allow, the one whose workgroups
    // fill the rounds of 256 best (then the fewest splits, which the finalize
    // has to add).
    constexpr int64_t kCus = 256;
    const int64_t s_lo = std::max<int64_t>((kblocks + kMaxSteps - 1) / kMaxSteps, (kCus + tiles - 1) / tiles);
    int64_t best_per = (kblocks + s_lo - 1) / s_lo;
    double best_eff = -1.0;
    for (int64_t per = std::max<int64_t>(1, best_per); per >= 1 && per >= best_per / 2; --per) {
      // the grid deals splits to the 8 XCDs (whole groups of 8 splits)
      const int64_t sp = (kblocks + per - 1) / per, wg = sp * tiles, slots = ((sp + 7) / 8) * 8 * tiles;
      const double eff = (double)wg / (double)(((slots + kCus - 1) / kCus) * kCus);
      if (eff > best_eff + 1e-9) {
        best_eff = eff;
        best_per = per;
      }
    }
    pl.kchunk = std::max<int64_t>(1, best_per) * kGramK;
    pl.splits = (int32_t)std::max<int64_t>(1, (len + pl.kchunk - 1) / pl.kchunk);
  }
  pl.ws_bytes = (size_t)pl.splits * n_batch * ((size_t)n_recv * n_send + n_recv + n_send) * sizeof(float);
  return pl;
}

template <int NTH>
static void gram_launch(const CosineArgs& a, hipStream_t st) {
  // two steps in flight where the second register set fits beside the accumulators
  constexpr int DEPTH = NTH <= 8 ? 2 : 1;
  const int n_rtiles = (a.n_recv + kGramRows - 1) / kGramRows;
  dim3 grid(kXcds * ((a.splits + kXcds - 1) / kXcds) * n_rtiles, a.n_batch);
  {
    KernelTimer kt_("k_gram_bf16", st);
    hipLaunchKernelGGL((k_gram_bf16<NTH, DEPTH>), grid, dim3(kGramThreads), 0, st, a);
  }
}

hipError_t launch_cosine(const CosineArgs& a, hipStream_t st) {
  if (a.n_batch == 0 || a.n_recv == 0) return hipSuccess;
  if (a.bf16) {
    const int nth = (a.n_send + 31) / 32;  // sender tiles of 32
    if (nth <= 1) gram_launch<1>(a, st);
    else if (nth <= 2) gram_launch<2>(a, st);
    else if (nth <= 4) gram_launch<4>(a, st);
    else if (nth <= 8) gram_launch<8>(a, st);
    else if (nth <= 11) gram_launch<11>(a, st);
    else gram_launch<12>(a, st);
  } else {
    { KernelTimer kt_("k_gram_f32", st); hipLaunchKernelGGL(k_gram_f32, dim3(a.n_send, a.n_recv, a.n_batch), dim3(256), 0, st, a); }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  { KernelTimer kt_("k_cos_finalize", st); hipLaunchKernelGGL(k_cos_finalize, dim3(a.n_recv, a.n_batch), dim3(kFinThreads), 0, st, a); }
  return hipGetLastError();
}

}  // namespace cma
