// Head mapping by cosine similarity of flattened maps (IAM Methods 1 and 4).
//
// The cosine matrix is a Gram product R S^T over the map length with the row
// norms on the side. It runs as a split-K bf16 MFMA GEMM: a workgroup (8 waves)
// owns 128 receiver maps and one K-chunk and holds the partial dot products of
// its 128 maps against all sender maps in registers (wave = 32 receivers x one
// half of the senders). Each 64-element K-step is software-pipelined: while the
// step's products run, the next step's receiver operands (straight from HBM,
// each receiver map read once) and sender slice (into registers, then into the
// other half of a double-buffered LDS slice shared by all waves) are in flight.
// Partial sums of each split go to a workspace and a finalize kernel adds them
// in a fixed order (deterministic), forms the cosines and takes argmax (lowest
// index on ties) and margin.
#include "kernels.hpp"

namespace cma {

constexpr int kGramRows = 128;     // receiver maps per workgroup
constexpr int kGramK = 64;         // K elements per step
constexpr int kGramThreads = 512;  // 8 waves = 4 groups of 32 receivers x 2 sender halves
constexpr int kMaxSteps = 64;      // K-steps of one split (4096 elements)

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

template <int NTH>  // sender tiles of 16 per half (n_send <= 32 * NTH)
__global__ __launch_bounds__(kGramThreads) void k_gram_bf16(CosineArgs a) {
  constexpr int SROWS = 32 * NTH;                                  // staged sender rows
  constexpr int SCH = SROWS * 8;                                   // 16-byte chunks per slice
  constexpr int SPT = (SCH + kGramThreads - 1) / kGramThreads;     // chunks per thread
  __shared__ __attribute__((aligned(16))) u32x4 sb[2][SCH];
  const int b = blockIdx.y;
  const int n_rtiles = (a.n_recv + kGramRows - 1) / kGramRows;
  // Workgroup id i runs on XCD i % 8. Split sp goes to XCD sp % 8 with all its
  // receiver tiles in consecutive slots there, so the tiles of a split run
  // together and share its sender slice through that XCD's L2.
  const int xcd = blockIdx.x % kXcds, m = blockIdx.x / kXcds;
  const int sp = xcd + kXcds * (m / n_rtiles), rt = m % n_rtiles;
  if (sp >= a.splits) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int p = lane & 15, qd = lane >> 4;
  const int rg = wave & 3, sh = wave >> 2;  // receiver group, sender half
  const int64_t k_beg = (int64_t)sp * a.kchunk;
  const int64_t k_end = min(a.len, k_beg + a.kchunk);
  const int nsteps = (int)((k_end - k_beg + kGramK - 1) / kGramK);
  const uint16_t* recv = reinterpret_cast<const uint16_t*>(a.recv) + (int64_t)b * a.rb;
  const uint16_t* send = reinterpret_cast<const uint16_t*>(a.send) + (int64_t)b * a.sb;
  const int row0 = rt * kGramRows + 32 * rg;

  f32x4 acc[2][NTH];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTH; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Squared norms in two levels: a step's squares are summed apart, added to an
  // inner running sum that is folded into the outer one every 16 steps. A single
  // long fp32 chain would drop the many tiny squares of a probability map's tail
  // once the sum has grown (a systematic underestimate, which biases the cosine).
  float rn[2] = {0.f, 0.f}, rn_in[2] = {0.f, 0.f};
  float sn = 0.f, sn_in = 0.f;
  // sender rows whose norms this workgroup accumulates (one per thread): the
  // receiver tiles of a split share the rows out
  const int s_per = (a.n_send + n_rtiles - 1) / n_rtiles;
  const int srow = rt * s_per + tid;
  const bool s_mine = tid < s_per && srow < a.n_send;

  const uint16_t* arow[2];
  bool aok[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int row = row0 + 16 * mt + p;
    aok[mt] = row < a.n_recv;
    arow[mt] = recv + (int64_t)(aok[mt] ? row : 0) * a.rh;
  }
  // The loads of a full step carry no branch, so the compiler's waits for the
  // prefetched registers stay exact: rows past the end read a valid row, and
  // what they produce (products in rows or columns past the end, their norms)
  // is never stored. A last, partial step uses element-guarded loads.
  // receiver operand of step st: lane (p, qd) holds k = 32 ks + 8 qd .. + 7 of its rows
  auto load_a = [&](int st, u32x4 (&av)[2][2], auto guarded) __attribute__((always_inline)) {
    const int64_t k0 = k_beg + (int64_t)st * kGramK;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int64_t j0 = k0 + 32 * ks + 8 * qd;
        if constexpr (decltype(guarded)::value) {
          u32x4 x = {0u, 0u, 0u, 0u};
          if (aok[mt]) x = ldg16_guard(arow[mt], j0, k_end);
          av[mt][ks] = x;
        } else {
          av[mt][ks] = ldg16(arow[mt] + j0);
        }
      }
  };
  // sender slice of step st: chunk x = tid + 512 i is (row x / 8, LDS slot x % 8)
  auto load_s = [&](int st, u32x4 (&sv)[SPT], auto guarded) __attribute__((always_inline)) {
    const int64_t k0 = k_beg + (int64_t)st * kGramK;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int x = tid + kGramThreads * i, row = x >> 3, slot = x & 7;
      const int ch = slot ^ ((row >> 1) & 7);
      const bool ok = x < SCH && row < a.n_send;
      const uint16_t* srow_p = send + (int64_t)min(row, a.n_send - 1) * a.sh;
      if constexpr (decltype(guarded)::value) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok) v = ldg16_guard(srow_p, k0 + 8 * ch, k_end);
        sv[i] = v;
      } else {
        sv[i] = ldg16(srow_p + k0 + 8 * ch);
      }
    }
  };
  auto store_s = [&](const u32x4 (&sv)[SPT], int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int x = tid + kGramThreads * i;
      if (x < SCH) sb[buf][x] = sv[i];  // slot order: x = row * 8 + slot
    }
  };
  // one step's work on the slice in LDS buffer buf and the receiver operand av
  auto compute = [&](int st, int buf, const u32x4 (&av)[2][2]) __attribute__((always_inline)) {
    // receiver norms (one sender half does it)
    if (sh == 0) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        float t = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int e = 0; e < 4; ++e) t = sq2(av[mt][ks][e], t);
        rn_in[mt] += t;
      }
    }
    // sender norms of this workgroup's share of the rows, in element order
    if (s_mine) {
      float t = 0.0f;
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        const u32x4 v = sb[buf][sslot(srow, ch)];
#pragma unroll
        for (int e = 0; e < 4; ++e) t = sq2(v[e], t);
      }
      sn_in += t;
    }
    if (((st + 1) & 15) == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        rn[u] += rn_in[u];
        rn_in[u] = 0.0f;
      }
      sn += sn_in;
      sn_in = 0.0f;
    }
    // products: B operand lane (p, qd) = sender row 16 nt + p, k = 32 ks + 8 qd .. + 7
#pragma unroll
    for (int nt = 0; nt < NTH; ++nt) {
      const int srow_b = 16 * (sh * NTH + nt) + p;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 bv = sb[buf][sslot(srow_b, 4 * ks + qd)];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma16(as_bf16x8(av[mt][ks]), as_bf16x8(bv), acc[mt][nt]);
      }
    }
  };

  using Fast = std::integral_constant<bool, false>;
  using Guarded = std::integral_constant<bool, true>;
  const int nfull = (int)((k_end - k_beg) / kGramK);  // steps with all 64 elements inside the chunk
  u32x4 acur[2][2], anext[2][2], sv[SPT];
  if (nfull > 0) {
    load_s(0, sv, Fast{});
    load_a(0, acur, Fast{});
    store_s(sv, 0);
  }
  __syncthreads();
  for (int st = 0; st < nfull; ++st) {
    const int buf = st & 1;
    // the next full step's operands (clamped at the end: a harmless reload)
    const int nx = min(st + 1, nfull - 1);
    load_s(nx, sv, Fast{});
    load_a(nx, anext, Fast{});
    compute(st, buf, acur);
    store_s(sv, buf ^ 1);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acur[mt][ks] = anext[mt][ks];
    __syncthreads();
  }
  if (nfull < nsteps) {
    // the partial last step
    const int buf = nfull & 1;
    load_s(nfull, sv, Guarded{});
    load_a(nfull, acur, Guarded{});
    store_s(sv, buf);
    __syncthreads();
    compute(nfull, buf, acur);
  }

#pragma unroll
  for (int u = 0; u < 2; ++u) rn[u] += rn_in[u];
  sn += sn_in;
  // partial dot products: D[m = 4qd + v][n = p]
  float* part = a.part + ((int64_t)sp * a.n_batch + b) * a.n_recv * a.n_send;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTH; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row0 + 16 * mt + 4 * qd + v, col = 16 * (sh * NTH + nt) + p;
        if (row < a.n_recv && col < a.n_send) part[(int64_t)row * a.n_send + col] = acc[mt][nt][v];
      }
  if (sh == 0) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float x = rn[mt];
      x += xor_lane(x, 16);
      x += xor_lane(x, 32);
      const int row = row0 + 16 * mt + p;
      if (qd == 0 && row < a.n_recv) a.rnorm[((int64_t)sp * a.n_batch + b) * a.n_recv + row] = x;
    }
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
  const int n_rtiles = (a.n_recv + kGramRows - 1) / kGramRows;
  dim3 grid(kXcds * ((a.splits + kXcds - 1) / kXcds) * n_rtiles, a.n_batch);
  { KernelTimer kt_("k_gram_bf16", st); hipLaunchKernelGGL((k_gram_bf16<NTH>), grid, dim3(kGramThreads), 0, st, a); }
}

hipError_t launch_cosine(const CosineArgs& a, hipStream_t st) {
  if (a.n_batch == 0 || a.n_recv == 0) return hipSuccess;
  if (a.bf16) {
    const int nth = (a.n_send + 31) / 32;  // sender tiles of 16 per half
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
