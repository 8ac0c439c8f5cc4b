// Two-phase block-sparse compression of causal maps (MapFlow, storage and
// execution): phase 1 gathers 64x64 block statistics in one QK^T sweep per
// block-row and selects the blocks to keep; phase 2 recomputes only the kept
// blocks and writes them. The dense map is never formed.
//
// Phase 1 (k_block_stats): per block-row, 8 waves sweep the key blocks (two
// query tiles x four key phases). For every (query, key block) the online
// softmax leaves a partial sum relative to the running max at that block; both
// go to LDS. After the sweep the running statistics of the four key phases are
// merged into each query's final (max, sum), and the mass of block c is
//   mass_c = sum_i partial_ic * 2^(max_ic - max_i) / sum_i
// added over the 64 query rows in a fixed order. Selection (normalise by the
// block-row total, order largest first with ties to the lower column, keep the
// shortest prefix whose running sum reaches tau) runs in the same workgroup: a
// bitonic sort in LDS and a sequential running sum.
// Scan (k_bsr_scan): exclusive scan of kept counts -> row_ptr, nnz.
// Phase 2 (k_block_extract): per block-row, recompute the kept blocks' scores,
// p = 2^(t - lse2) and store bf16 blocks and their column indices.
#include "kernels.hpp"
#include "score.hpp"

namespace cma {

template <int D>
__global__ __launch_bounds__(512) void k_block_stats(CompressArgs a) {
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  const int R = a.nrb_max;               // LDS arrays are [64][R]
  float* P = dyn;                        // partial sums
  float* MX = dyn + 64 * R;              // running max at each block
  __shared__ float sm[4][64], sl[4][64];
  __shared__ float Mrow[64], Lrow[64];
  __shared__ float mass[kMaxBlockRows];
  __shared__ unsigned long long keys[kMaxBlockRows];
  __shared__ uint32_t kept[kWords];
  __shared__ int kcount;

  const int h = blockIdx.z, s = blockIdx.y;
  const int r = (int)gridDim.x - 1 - (int)blockIdx.x;
  const int32_t n = seq_len_q(a.vl, s);
  if (!seq_ok(a.vl, s, n, n) || 64 * r >= n) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int qt = wave & 1, kp = wave >> 1;
  const int iloc = 32 * qt + (lane & 31);
  const int i = 64 * r + iloc;
  const bool valid = i < n;
  const uint16_t* qrow = a.q + ((int64_t)h * a.vl.total_q + a.vl.cu_q[s] + i) * D;
  const uint16_t* kseq = a.k + ((int64_t)h * a.vl.total_k + a.vl.cu_k[s]) * D;
  const float scale_l2 = a.scale[h] * kLog2e;
  const float bias_l2 = a.bias ? a.bias[h] * kLog2e : 0.0f;

  QOperand<D> qop;
  load_query<D>(qop, qrow, valid);
  f32x16 acc[2];
  float t[32];
  float m = -INFINITY, l = 0.0f;
  for (int c = kp; c <= r; c += 4) {
    score_block<D>(acc, qop, kseq, 64 * c, n);
    logits_block(t, acc, 64 * c, valid ? i : -1, scale_l2, bias_l2);
    const float part = online_update(t, m, l);
    if (lane < 32) {
      P[iloc * R + c] = part;
      MX[iloc * R + c] = m;
    }
  }
  if (lane < 32) {
    sm[kp][iloc] = m;
    sl[kp][iloc] = l;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int q = threadIdx.x;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][q]);
    float L = 0.0f;
    for (int w = 0; w < 4; ++w)
      if (sm[w][q] != -INFINITY) L += sl[w][q] * exp2f_fast(sm[w][q] - M);
    Mrow[q] = M;
    Lrow[q] = L;
    const int iq = 64 * r + q;
    if (iq < n) {
      const int64_t tok = (int64_t)h * a.vl.total_q + a.vl.cu_q[s] + iq;
      a.lse2[tok] = M + log2f_fast(L);
      if (a.row_stats) {
        a.row_stats[2 * tok] = M * kLn2;
        a.row_stats[2 * tok + 1] = L;
      }
    }
  }
  if (threadIdx.x < kWords) kept[threadIdx.x] = 0u;
  __syncthreads();
  const int nrows = min(64, n - 64 * r);
  for (int c = threadIdx.x; c <= r; c += 512) {
    float x = 0.0f;
    for (int q = 0; q < nrows; ++q) x += P[q * R + c] * exp2f_fast(MX[q * R + c] - Mrow[q]) / Lrow[q];
    mass[c] = x;
  }
  __syncthreads();

  int32_t roff;
  int64_t tri_off;
  block_offsets(a.vl, s, roff, tri_off);
  const int64_t g = (int64_t)h * a.n_block_rows + roff + r;
  if (a.block_mass) {
    int32_t r_all;
    int64_t n_tri;  // blocks per head over all sequences
    block_offsets(a.vl, a.vl.n_seqs, r_all, n_tri);
    float* bm = a.block_mass + (int64_t)h * n_tri + tri_off + (int64_t)r * (r + 1) / 2;
    for (int c = threadIdx.x; c <= r; c += 512) bm[c] = mass[c];
  }
  const int nb = r + 1;
  if (a.tau >= 1.0f) {
    for (int c = threadIdx.x; c < kMaxBlockRows; c += 512)
      if (c < nb) atomicOr(&kept[c >> 5], 1u << (c & 31));
    if (threadIdx.x == 0) kcount = nb;
  } else {
    // total mass: one wave, strided partial sums then a fixed butterfly
    if (wave == 0) {
      float x = 0.0f;
      for (int c = lane; c < nb; c += 64) x += mass[c];
      for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
      if (lane == 0) sm[0][0] = x;
    }
    __syncthreads();
    const float total = sm[0][0];
    int ns = 1;
    while (ns < nb) ns <<= 1;
    for (int c = threadIdx.x; c < ns; c += 512) {
      if (c < nb) {
        const float w = mass[c] / total;
        keys[c] = ((unsigned long long)(0xffffffffu - __float_as_uint(w)) << 32) | (uint32_t)c;
      } else {
        keys[c] = ~0ull;
      }
    }
    __syncthreads();
    // bitonic sort, ascending key = weight descending, column ascending
    for (int size = 2; size <= ns; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int x = threadIdx.x; x < ns / 2; x += 512) {
          const int lo = 2 * stride * (x / stride) + (x % stride);
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const unsigned long long kl = keys[lo], kh = keys[hi];
          if ((kl > kh) == up) {
            keys[lo] = kh;
            keys[hi] = kl;
          }
        }
        __syncthreads();
      }
    }
    if (threadIdx.x == 0) {
      float cum = 0.0f;
      int k = nb;
      for (int x = 0; x < nb; ++x) {
        const int c = (int)(keys[x] & 0xffffffffu);
        cum += mass[c] / total;
        if (cum >= a.tau) {
          k = x + 1;
          break;
        }
      }
      kcount = k;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < kcount; x += 512) {
      const int c = (int)(keys[x] & 0xffffffffu);
      atomicOr(&kept[c >> 5], 1u << (c & 31));
    }
  }
  __syncthreads();
  if (threadIdx.x < kWords) a.kept[g * kWords + threadIdx.x] = kept[threadIdx.x];
  if (threadIdx.x == 0) a.counts[g] = kcount;
}

// Exclusive scan of the kept counts (one workgroup). Deterministic (integers).
__global__ __launch_bounds__(1024) void k_bsr_scan(const int32_t* counts, int64_t n, int32_t* row_ptr,
                                                   int32_t* nnz) {
  __shared__ int64_t part[1024];
  const int t = threadIdx.x;
  const int64_t chunk = (n + 1023) / 1024;
  const int64_t b0 = t * chunk, b1 = min(n, b0 + chunk);
  int64_t sum = 0;
  for (int64_t x = b0; x < b1; ++x) sum += counts[x];
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int64_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int64_t run = part[t] - sum;  // exclusive prefix of this chunk
  for (int64_t x = b0; x < b1; ++x) {
    row_ptr[x] = (int32_t)run;
    run += counts[x];
  }
  if (t == 1023) {
    row_ptr[n] = (int32_t)part[1023];
    nnz[0] = (int32_t)part[1023];
  }
}

template <int D>
__global__ __launch_bounds__(512) void k_block_extract(CompressArgs a) {
  __shared__ int cols[kMaxBlockRows];
  __shared__ int ncols;
  const int h = blockIdx.z, s = blockIdx.y;
  const int r = (int)gridDim.x - 1 - (int)blockIdx.x;
  const int32_t n = seq_len_q(a.vl, s);
  if (!seq_ok(a.vl, s, n, n) || 64 * r >= n) return;
  if ((int64_t)a.nnz[0] > a.capacity) return;
  int32_t roff;
  int64_t tri_off;
  block_offsets(a.vl, s, roff, tri_off);
  const int64_t g = (int64_t)h * a.n_block_rows + roff + r;
  if (threadIdx.x == 0) {
    int k = 0;
    for (int w = 0; w < kWords; ++w) {
      uint32_t bits = a.kept[g * kWords + w];
      while (bits) {
        const int b = __builtin_ctz(bits);
        cols[k++] = 32 * w + b;
        bits &= bits - 1;
      }
    }
    ncols = k;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int qt = wave & 1, kp = wave >> 1;
  const int iloc = 32 * qt + (lane & 31);
  const int i = 64 * r + iloc;
  const bool valid = i < n;
  const int half = lane >> 5;
  const uint16_t* qrow = a.q + ((int64_t)h * a.vl.total_q + a.vl.cu_q[s] + i) * D;
  const uint16_t* kseq = a.k + ((int64_t)h * a.vl.total_k + a.vl.cu_k[s]) * D;
  const float scale_l2 = a.scale[h] * kLog2e;
  const float bias_l2 = a.bias ? a.bias[h] * kLog2e : 0.0f;
  const float lse = valid ? a.lse2[(int64_t)h * a.vl.total_q + a.vl.cu_q[s] + i] : 0.0f;
  const int64_t base = a.row_ptr[g];
  QOperand<D> qop;
  load_query<D>(qop, qrow, valid);
  f32x16 acc[2];
  float t[32];
  for (int x = kp; x < ncols; x += 4) {
    const int c = cols[x];
    score_block<D>(acc, qop, kseq, 64 * c, n);
    logits_block(t, acc, 64 * c, valid ? i : -1, scale_l2, bias_l2);
    uint16_t* blk = a.vals + (base + x) * (int64_t)(kBlock * kBlock);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = valid ? exp2f_fast(t[kt * 16 + 4 * gq + e] - lse) : 0.0f;
        const int j = 32 * kt + 8 * gq + 4 * half;
        u32x2 w = {pack2bf(p[0], p[1]), pack2bf(p[2], p[3])};
        *reinterpret_cast<u32x2*>(blk + blk_off(iloc, j)) = w;
      }
    if (qt == 0 && lane == 0) a.col_idx[base + x] = c;
  }
}

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t value) {
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (x < n) p[x] = value;
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  { KernelTimer kt_("k_fill_i32", st); hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, value); }
  return hipGetLastError();
}

size_t compress_ws_bytes(int32_t n_heads, int32_t n_block_rows, int64_t total_q) {
  const size_t g = (size_t)n_heads * n_block_rows;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(g * sizeof(int32_t)) + al(g * kWords * sizeof(uint32_t)) +
         al((size_t)n_heads * total_q * sizeof(float));
}

template <int D>
static hipError_t compress_impl(const CompressArgs& a, hipStream_t st) {
  dim3 grid(a.nrb_max, a.vl.n_seqs, a.n_heads);
  const size_t lds = (size_t)2 * 64 * a.nrb_max * sizeof(float);
  hipError_t e0 = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_block_stats<D>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e0 != hipSuccess) return e0;
  { KernelTimer kt_("k_block_stats", st); hipLaunchKernelGGL((k_block_stats<D>), grid, dim3(512), lds, st, a); }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    KernelTimer kt_("k_bsr_scan", st);
    hipLaunchKernelGGL(k_bsr_scan, dim3(1), dim3(1024), 0, st, a.counts,
                       (int64_t)a.n_heads * a.n_block_rows, a.row_ptr, a.nnz);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  { KernelTimer kt_("k_block_extract", st); hipLaunchKernelGGL((k_block_extract<D>), grid, dim3(512), 0, st, a); }
  return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs& a, int d, hipStream_t st) {
  if (a.n_heads == 0 || a.vl.n_seqs == 0 || a.nrb_max == 0) {
    return hipSuccess;
  }
  return d == 64 ? compress_impl<64>(a, st) : compress_impl<128>(a, st);
}

}  // namespace cma
