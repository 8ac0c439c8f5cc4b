// Head mapping by cosine similarity of flattened maps (IAM Methods 1 and 4).
//
// The cosine matrix is a Gram product R S^T over the map length with the row
// norms on the side. It runs as a split-K bf16 MFMA GEMM: a workgroup owns 128
// receiver maps and one K-chunk, holds the partial dot products of its 128 maps
// against all sender maps in registers, stages the sender slice through LDS
// (shared by its 4 waves) and streams its own receiver rows straight from HBM,
// so each receiver map is read once. Partial sums of each split go to a
// workspace and a finalize kernel adds them in a fixed order (deterministic),
// forms the cosines and takes argmax (lowest index on ties) and margin.
#include "kernels.hpp"

namespace cma {

constexpr int kGramRows = 128;  // receiver maps per workgroup
constexpr int kGramK = 64;      // K elements per step
constexpr int kSbStride = 72;   // padded LDS row (bf16) of the staged sender slice
constexpr int kMaxSteps = 64;   // K-steps of one split (4096 elements)

template <int NT>  // sender tiles of 16 (n_send <= 16 * NT)
__global__ __launch_bounds__(256) void k_gram_bf16(CosineArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sb[NT * 16 * kSbStride];
  const int n_rtiles = (a.n_recv + kGramRows - 1) / kGramRows;
  const int b = blockIdx.y;
  const int rt = blockIdx.x / a.splits, sp = blockIdx.x % a.splits;
  (void)n_rtiles;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int p = lane & 15, qd = lane >> 4;
  const int64_t k_beg = (int64_t)sp * a.kchunk;
  const int64_t k_end = min(a.len, k_beg + a.kchunk);
  const uint16_t* recv = reinterpret_cast<const uint16_t*>(a.recv) + (int64_t)b * a.rb;
  const uint16_t* send = reinterpret_cast<const uint16_t*>(a.send) + (int64_t)b * a.sb;
  const int row0 = rt * kGramRows + 32 * wave;

  f32x4 acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Squared norms in two levels: a step's squares are summed apart, added to an
  // inner running sum that is folded into the outer one every 16 steps. A single
  // long fp32 chain would drop the many tiny squares of a probability map's tail
  // once the sum has grown (a systematic underestimate, which biases the cosine).
  float rn[2] = {0.f, 0.f}, rn_in[2] = {0.f, 0.f};
  float sn[2] = {0.f, 0.f}, sn_in[2] = {0.f, 0.f};  // sender rows threadIdx.x, threadIdx.x + 256
  int step = 0;

  const uint16_t* arow[2];
  bool aok[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int row = row0 + 16 * mt + p;
    aok[mt] = row < a.n_recv;
    arow[mt] = recv + (int64_t)(aok[mt] ? row : 0) * a.rh;
  }

  for (int64_t k0 = k_beg; k0 < k_end; k0 += kGramK) {
    // stage the sender slice [NT*16 rows][64]
    for (int x = threadIdx.x; x < NT * 16 * 8; x += 256) {
      const int row = x >> 3, ch = x & 7;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (row < a.n_send) val = ldg16_guard(send + (int64_t)row * a.sh, k0 + 8 * ch, k_end);
      *reinterpret_cast<u32x4*>(&sb[row * kSbStride + 8 * ch]) = val;
    }
    // receiver operand straight from memory
    u32x4 av[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (aok[mt]) x = ldg16_guard(arow[mt], k0 + 32 * ks + 8 * qd, k_end);
        av[mt][ks] = x;
      }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float t = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(av[mt][ks][e] << 16);
          const float hi = __uint_as_float(av[mt][ks][e] & 0xffff0000u);
          t = fmaf(lo, lo, fmaf(hi, hi, t));
        }
      rn_in[mt] += t;
    }
    __syncthreads();
    if (rt == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int row = threadIdx.x + 256 * u;
        if (row < NT * 16) {
          const uint16_t* srow = &sb[row * kSbStride];
          float t = 0.0f;
          for (int e = 0; e < kGramK; ++e) {
            const float x = bf2f(srow[e]);
            t = fmaf(x, x, t);
          }
          sn_in[u] += t;
        }
      }
    }
    if ((++step & 15) == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        rn[u] += rn_in[u];
        sn[u] += sn_in[u];
        rn_in[u] = sn_in[u] = 0.0f;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 bv = *reinterpret_cast<const u32x4*>(&sb[(16 * nt + p) * kSbStride + 32 * ks + 8 * qd]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma16(as_bf16x8(av[mt][ks]), as_bf16x8(bv), acc[mt][nt]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int u = 0; u < 2; ++u) {
    rn[u] += rn_in[u];
    sn[u] += sn_in[u];
  }
  // partial dot products: D[m = 4qd + v][n = p]
  float* part = a.part + ((int64_t)sp * a.n_batch + b) * a.n_recv * a.n_send;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row0 + 16 * mt + 4 * qd + v, col = 16 * nt + p;
        if (row < a.n_recv && col < a.n_send) part[(int64_t)row * a.n_send + col] = acc[mt][nt][v];
      }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    float x = rn[mt];
    x += xor_lane(x, 16);
    x += xor_lane(x, 32);
    const int row = row0 + 16 * mt + p;
    if (qd == 0 && row < a.n_recv) a.rnorm[((int64_t)sp * a.n_batch + b) * a.n_recv + row] = x;
  }
  if (rt == 0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = threadIdx.x + 256 * u;
      if (row < a.n_send) a.snorm[((int64_t)sp * a.n_batch + b) * a.n_send + row] = sn[u];
    }
  }
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

// one wave per (receiver map, problem)
__global__ __launch_bounds__(64) void k_cos_finalize(CosineArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  float rn = 0.f;
  for (int sp = 0; sp < a.splits; ++sp) rn += a.rnorm[((int64_t)sp * a.n_batch + b) * a.n_recv + h];
  const float rs = sqrtf(rn);
  float v1 = -INFINITY, v2 = -INFINITY;
  int i1 = 0x7fffffff, i2 = 0x7fffffff;
  for (int j = lane; j < a.n_send; j += 64) {
    float dot = 0.f, sn = 0.f;
    for (int sp = 0; sp < a.splits; ++sp) {
      dot += a.part[(((int64_t)sp * a.n_batch + b) * a.n_recv + h) * a.n_send + j];
      sn += a.snorm[((int64_t)sp * a.n_batch + b) * a.n_send + j];
    }
    const float den = rs * sqrtf(sn);
    const float c = den > 0.f ? dot / den : 0.f;
    if (a.cos) a.cos[((int64_t)b * a.n_recv + h) * a.n_send + j] = c;
    if (better(c, j, v1, i1)) {
      v2 = v1; i2 = i1; v1 = c; i1 = j;
    } else if (better(c, j, v2, i2)) {
      v2 = c; i2 = j;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float ov1 = __shfl_xor(v1, off, 64), ov2 = __shfl_xor(v2, off, 64);
    const int oi1 = __shfl_xor(i1, off, 64), oi2 = __shfl_xor(i2, off, 64);
    // merge the two top-2 lists
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
  if (lane == 0) {
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
    // enough splits to fill the chip, and at most kMaxSteps K-steps per split so
    // that each partial dot product is a short fp32 accumulation chain
    int64_t splits = (512 + tiles - 1) / tiles;
    splits = std::max<int64_t>(splits, (kblocks + kMaxSteps - 1) / kMaxSteps);
    splits = std::max<int64_t>(1, std::min<int64_t>(splits, kblocks));
    const int64_t per = (kblocks + splits - 1) / splits;
    pl.kchunk = std::max<int64_t>(1, per) * kGramK;
    pl.splits = (int32_t)std::max<int64_t>(1, (len + pl.kchunk - 1) / pl.kchunk);
  }
  pl.ws_bytes = (size_t)pl.splits * n_batch * ((size_t)n_recv * n_send + n_recv + n_send) * sizeof(float);
  return pl;
}

template <int NT>
static void gram_launch(const CosineArgs& a, hipStream_t st) {
  const int n_rtiles = (a.n_recv + kGramRows - 1) / kGramRows;
  dim3 grid(n_rtiles * a.splits, a.n_batch);
  { KernelTimer kt_("k_gram_bf16", st); hipLaunchKernelGGL((k_gram_bf16<NT>), grid, dim3(256), 0, st, a); }
}

hipError_t launch_cosine(const CosineArgs& a, hipStream_t st) {
  if (a.n_batch == 0 || a.n_recv == 0) return hipSuccess;
  if (a.bf16) {
    const int nt = (a.n_send + 15) / 16;
    if (nt <= 1) gram_launch<1>(a, st);
    else if (nt <= 2) gram_launch<2>(a, st);
    else if (nt <= 4) gram_launch<4>(a, st);
    else if (nt <= 8) gram_launch<8>(a, st);
    else if (nt <= 12) gram_launch<12>(a, st);
    else if (nt <= 16) gram_launch<16>(a, st);
    else if (nt <= 21) gram_launch<21>(a, st);
    else gram_launch<24>(a, st);
  } else {
    { KernelTimer kt_("k_gram_f32", st); hipLaunchKernelGGL(k_gram_f32, dim3(a.n_send, a.n_recv, a.n_batch), dim3(256), 0, st, a); }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  { KernelTimer kt_("k_cos_finalize", st); hipLaunchKernelGGL(k_cos_finalize, dim3(a.n_recv, a.n_batch), dim3(64), 0, st, a); }
  return hipGetLastError();
}

}  // namespace cma
