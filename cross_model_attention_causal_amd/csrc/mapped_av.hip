// Fused mapped attention x V (MapFlow, approach and storage-and-execution
// sections; IAM Method 4 for decode rows):  O_h = (sum_j M[h, j] A_j) V_h.
//
// Block-sparse source (k_mapped_av_bsr). A workgroup owns 32 query rows of one
// block-row and 16 receiver heads and walks the union of the sender heads' kept
// columns in ascending order. Per key block and 32-key half it
//   1. stages the 32 senders' 32x32 sub-blocks in LDS (zeros where a sender did
//      not keep the block),
//   2. mixes them on the matrix cores: for 16 positions at a time
//      D1[h, pos] = sum_j M[h, j] A_j[pos] is a 16x16x32 MFMA with M (split
//      into bf16 high and low parts, so the mix is accurate to ~2^-16) as the A
//      operand and the senders as the B operand, read with the transposing LDS
//      load so that each lane gets 8 senders of one position,
//   3. writes the mixed maps B_h (bf16) to LDS and multiplies them into V_h with
//      32x32x16 MFMAs, accumulating O in fp32 registers.
// V is read as a transposed copy (key index contiguous) so that the V operand
// comes straight from memory with 16-byte loads. The mixed map never leaves LDS.
//
// Dense source (k_mapped_av_dense): VALU kernel for small problems and decode
// rows: one workgroup per (query row, sequence, receiver head); only the
// nonzero mixing weights are visited, so a one-hot M reads one sender row.
#include "kernels.hpp"

namespace cma {

constexpr int kHeadsPerWg = 16;
constexpr int kRowsPerWg = 32;
constexpr int kSendPerStep = 32;
constexpr int kSendStride = 1056;  // bf16 per staged sender: 32 rows x 32 + 32 pad
constexpr int kBStride = 40;       // bf16 per mixed-map row (32 + 8 pad)
constexpr int kBHead = 1288;       // bf16 per mixed-map head (32 rows x 40 + 8 pad)

// Vt[h][e][t] = V[h][t][e]; grid (ceil(total_k / 64), n_heads), 256 threads.
template <int D>
__global__ __launch_bounds__(256) void k_transpose_v(const uint16_t* __restrict__ v, uint16_t* __restrict__ vt,
                                                     int64_t total_k) {
  __shared__ uint16_t tile[64][D + 2];
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const uint16_t* src = v + ((int64_t)h * total_k) * D;
  for (int x = threadIdx.x; x < 64 * D; x += 256) {
    const int tt = x / D, e = x % D;
    tile[tt][e] = (t0 + tt < total_k) ? src[(t0 + tt) * D + e] : (uint16_t)0;
  }
  __syncthreads();
  uint16_t* dst = vt + (int64_t)h * D * total_k;
  for (int x = threadIdx.x; x < 64 * D; x += 256) {
    const int e = x / 64, tt = x % 64;
    if (t0 + tt < total_k) dst[(int64_t)e * total_k + t0 + tt] = tile[tt][e];
  }
}

// grid (2 * n_block_rows_max, n_seqs, ceil(n_recv / 16)), 256 threads (4 waves).
__global__ __launch_bounds__(256) void k_mapped_av_bsr(MappedAvArgs a) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(16))) uint16_t sbuf[kSendPerStep * kSendStride];
  __shared__ __attribute__((aligned(16))) uint16_t bbuf[kHeadsPerWg * kBHead];
  __shared__ int cur[kSendPerStep], endp[kSendPerStep], curcol[kSendPerStep];
  __shared__ int cnext;

  const int s = blockIdx.y, hg = blockIdx.z;
  const int slot = (int)gridDim.x - 1 - (int)blockIdx.x;  // longest block-rows first
  const int r = slot >> 1, rh = slot & 1;
  const int32_t n = seq_len_q(a.vl, s);
  if (!seq_ok(a.vl, s, n, n) || 64 * r + kRowsPerWg * rh >= n) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int32_t roff;
  int64_t tri;
  block_offsets(a.vl, s, roff, tri);

  // mixing weights, A operand of 16x16x32: lane (p = lane%16, q = lane/16) holds
  // M[hg*16 + p][8q + e]; high and low bf16 parts.
  bf16x8 mhi, mlo;
  {
    const int p = lane & 15, q = lane >> 4;
    const int h = hg * kHeadsPerWg + p;
    const float* Ms = a.M + (int64_t)s * a.M_stride;
    u32x4 hi, lo;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      float x[2], xh[2], xl[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = 8 * q + 2 * e2 + u;
        x[u] = (h < a.n_recv && j < a.n_send) ? Ms[(int64_t)h * a.n_send + j] : 0.0f;
        xh[u] = bf2f(f2bf(x[u]));
        xl[u] = x[u] - xh[u];
      }
      hi[e2] = pack2bf(xh[0], xh[1]);
      lo[e2] = pack2bf(xl[0], xl[1]);
    }
    mhi = as_bf16x8(hi);
    mlo = as_bf16x8(lo);
  }
  if (threadIdx.x < kSendPerStep) {
    const int j = threadIdx.x;
    if (j < a.n_send) {
      const int64_t g = (int64_t)j * a.n_block_rows + roff + r;
      cur[j] = a.row_ptr[g];
      endp[j] = a.row_ptr[g + 1];
    } else {
      cur[j] = 0;
      endp[j] = 0;
    }
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[t][dt] = f32x16{};
  __syncthreads();

  const int64_t k0 = a.vl.cu_k[s];
  const int row_base = 64 * r + kRowsPerWg * rh;  // first query row (sequence-local)
  int cprev = -1;
  while (true) {
    if (wave == 0) {
      int v = 0x7fffffff;
      if (lane < kSendPerStep) {
        int cc = cur[lane];
        if (cprev >= 0 && cc < endp[lane] && curcol[lane] == cprev) ++cc;
        cur[lane] = cc;
        v = cc < endp[lane] ? a.col_idx[cc] : 0x7fffffff;
        curcol[lane] = v;
      }
      for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
      if (lane == 0) cnext = v;
    }
    __syncthreads();
    const int c = cnext;
    if (c == 0x7fffffff) break;
    cprev = c;
    for (int jh = 0; jh < 2; ++jh) {
      // 1. stage senders' rows [row_base, +32) x cols [32 jh, +32) of block (r, c)
      for (int x = threadIdx.x; x < kSendPerStep * 32 * 4; x += 256) {
        const int j = x >> 7, row = (x >> 2) & 31, ch = x & 3;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (curcol[j] == c) {
          const uint16_t* src = a.vals + (int64_t)cur[j] * (kBlock * kBlock) +
                                (kRowsPerWg * rh + row) * kBlock + 32 * jh + 8 * ch;
          val = ldg16(src);
        }
        *reinterpret_cast<u32x4*>(&sbuf[j * kSendStride + row * 32 + 8 * ch]) = val;
      }
      __syncthreads();
      // 2. mix on MFMA: tile tau covers row tau/2, keys 16*(tau%2) .. +15
      {
        const int q = lane >> 4, p = lane & 15;
        const int e = (lane >> 2) & 3, cc = lane & 3;
        for (int tau = wave; tau < 64; tau += 4) {
          const int row = tau >> 1, jb = 16 * (tau & 1);
          const uint16_t* b0 = &sbuf[(8 * q + e) * kSendStride + row * 32 + jb + 4 * cc];
          const uint16_t* b1 = b0 + 4 * kSendStride;
          lds_bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) lds_bf16x4*)(b0));
          lds_bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) lds_bf16x4*)(b1));
          u32x2 l2 = __builtin_bit_cast(u32x2, lo4), h2 = __builtin_bit_cast(u32x2, hi4);
          u32x4 bv = {l2[0], l2[1], h2[0], h2[1]};
          f32x4 d1 = {0.f, 0.f, 0.f, 0.f};
          d1 = mfma16(mhi, as_bf16x8(bv), d1);
          d1 = mfma16(mlo, as_bf16x8(bv), d1);
#pragma unroll
          for (int v = 0; v < 4; ++v) bbuf[(4 * q + v) * kBHead + row * kBStride + jb + p] = f2bf(d1[v]);
        }
      }
      __syncthreads();
      // 3. O += B_h V_h for this wave's 4 heads
      {
        const int n32 = lane & 31, q2 = lane >> 5;
        const int64_t kbase = 64 * c + 32 * jh;  // sequence-local key of this half
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int hh = 4 * wave + t;
          const int h = hg * kHeadsPerWg + hh;
          if (h >= a.n_recv) break;
          bf16x8 av[2];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            av[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(&bbuf[hh * kBHead + n32 * kBStride + 16 * ks + 8 * q2]));
          const uint16_t* vtb = a.vt + (int64_t)h * D * a.vl.total_k + k0;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const uint16_t* vrow = vtb + (int64_t)(32 * dt + n32) * a.vl.total_k;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              const u32x4 bv = ldg16_guard_any(vrow, kbase + 16 * ks + 8 * q2, n);
              acc[t][dt] = mfma32(av[ks], as_bf16x8(bv), acc[t][dt]);
            }
          }
        }
      }
    }
  }
  // epilogue: D[m = row][n = e]: row = 8(v/4) + 4 q2 + (v%4), e = 32 dt + lane%32
  const int n32 = lane & 31, q2 = lane >> 5;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int h = hg * kHeadsPerWg + 4 * wave + t;
    if (h >= a.n_recv) break;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = row_base + 8 * (v >> 2) + 4 * q2 + (v & 3);
        if (row >= n) continue;
        const int64_t o = ((int64_t)h * a.vl.total_q + a.vl.cu_q[s] + row) * D + 32 * dt + n32;
        if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o] = f2bf(acc[t][dt][v]);
        else reinterpret_cast<float*>(a.out)[o] = acc[t][dt][v];
      }
  }
}

// grid (max_q, n_seqs, n_recv), 256 threads.
template <int D, bool KEY_MAJOR>
__global__ __launch_bounds__(256) void k_mapped_av_dense(MappedAvArgs a) {
  constexpr int JS = 256 / D;  // key slots per pass
  __shared__ float bj[256];
  __shared__ float red[JS][D];
  __shared__ int nzi[64];
  __shared__ float nzw[64];
  __shared__ int nnzm;
  __shared__ float okm[D];  // key-major accumulators (one per feature)
  const int i = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const int32_t nq = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
  if (!seq_ok(a.vl, s, nq, nk) || i >= nq) return;
  const float* Ms = a.M + (int64_t)s * a.M_stride + (int64_t)h * a.n_send;
  if (threadIdx.x == 0) {
    int k = 0;
    for (int j = 0; j < a.n_send; ++j)
      if (Ms[j] != 0.0f) {
        nzi[k] = j;
        nzw[k] = Ms[j];
        ++k;
      }
    nnzm = k;
  }
  for (int f = threadIdx.x; f < D; f += 256) okm[f] = 0.0f;
  __syncthreads();
  const int last = nk - nq + i;
  const int64_t row_off = map_seq_off(a.vl, s, a.packed) + map_row_off(i, nq, nk, a.packed);
  const int e = threadIdx.x % D, js = threadIdx.x / D;
  const int64_t k0 = a.vl.cu_k[s];
  float acc = 0.0f;
  for (int j0 = 0; j0 <= last; j0 += 256) {
    const int j = j0 + threadIdx.x;
    float b = 0.0f;
    if (j <= last) {
      for (int u = 0; u < nnzm; ++u) {
        const int64_t idx = (int64_t)nzi[u] * a.head_stride + row_off + j;
        const float x = a.maps_bf16 ? bf2f(reinterpret_cast<const uint16_t*>(a.maps)[idx])
                                    : reinterpret_cast<const float*>(a.maps)[idx];
        b = fmaf(nzw[u], x, b);
      }
    }
    bj[threadIdx.x] = b;
    __syncthreads();
    const int jend = min(256, last + 1 - j0);
    if (!KEY_MAJOR) {
      for (int jj = js; jj < jend; jj += JS) {
        const int64_t vidx = ((int64_t)h * a.vl.total_k + k0 + j0 + jj) * D + e;
        const float vv = a.v_bf16 ? bf2f(reinterpret_cast<const uint16_t*>(a.v)[vidx])
                                  : reinterpret_cast<const float*>(a.v)[vidx];
        acc = fmaf(bj[jj], vv, acc);
      }
    } else {
      // key-major V: a wave walks features; its lanes cover consecutive keys
      const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
      for (int f = wave; f < D; f += 4) {
        const int64_t vrow = ((int64_t)h * D + f) * a.vl.total_k + k0 + j0;
        float part = 0.0f;
        for (int jj = lane; jj < jend; jj += 64) {
          const float vv = a.v_bf16 ? bf2f(reinterpret_cast<const uint16_t*>(a.v)[vrow + jj])
                                    : reinterpret_cast<const float*>(a.v)[vrow + jj];
          part = fmaf(bj[jj], vv, part);
        }
        for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
        if (lane == 0) okm[f] += part;
      }
    }
    __syncthreads();
  }
  red[js][e] = acc;
  __syncthreads();
  if (threadIdx.x < D) {
    float o = 0.0f;
    if (KEY_MAJOR) o = okm[threadIdx.x];
    else
      for (int u = 0; u < JS; ++u) o += red[u][threadIdx.x];
    const int64_t oi = ((int64_t)h * a.vl.total_q + a.vl.cu_q[s] + i) * D + threadIdx.x;
    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[oi] = f2bf(o);
    else reinterpret_cast<float*>(a.out)[oi] = o;
  }
}

__global__ void k_onehot(const int32_t* argmax, int64_t rows, int32_t n_send, float* M) {
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= rows * n_send) return;
  const int64_t row = x / n_send;
  const int j = (int)(x % n_send);
  M[x] = argmax[row] == j ? 1.0f : 0.0f;
}

hipError_t launch_mapped_av_dense(const MappedAvArgs& a, hipStream_t st) {
  if (a.n_recv == 0 || a.vl.n_seqs == 0 || a.max_q == 0) return hipSuccess;
  dim3 grid(a.max_q, a.vl.n_seqs, a.n_recv);
  if (a.v_key_major) {
    if (a.d == 64) { KernelTimer kt_("k_mapped_av_dense", st); hipLaunchKernelGGL((k_mapped_av_dense<64, true>), grid, dim3(256), 0, st, a); }
    else { KernelTimer kt_("k_mapped_av_dense", st); hipLaunchKernelGGL((k_mapped_av_dense<128, true>), grid, dim3(256), 0, st, a); }
  } else {
    if (a.d == 64) { KernelTimer kt_("k_mapped_av_dense", st); hipLaunchKernelGGL((k_mapped_av_dense<64, false>), grid, dim3(256), 0, st, a); }
    else { KernelTimer kt_("k_mapped_av_dense", st); hipLaunchKernelGGL((k_mapped_av_dense<128, false>), grid, dim3(256), 0, st, a); }
  }
  return hipGetLastError();
}

hipError_t launch_mapped_av_bsr(const MappedAvArgs& a, hipStream_t st) {
  if (a.n_recv == 0 || a.vl.n_seqs == 0 || a.max_q == 0) return hipSuccess;
  if (a.vl.total_k > 0 && !a.v_key_major) {
    dim3 tg((unsigned)((a.vl.total_k + 63) / 64), a.n_recv);
    {
      KernelTimer kt_("k_transpose_v", st);
      hipLaunchKernelGGL((k_transpose_v<128>), tg, dim3(256), 0, st,
                         reinterpret_cast<const uint16_t*>(a.v), a.vt, a.vl.total_k);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nrb = (a.max_q + 63) / 64;
  dim3 grid(2 * nrb, a.vl.n_seqs, (a.n_recv + kHeadsPerWg - 1) / kHeadsPerWg);
  { KernelTimer kt_("k_mapped_av_bsr", st); hipLaunchKernelGGL(k_mapped_av_bsr, grid, dim3(256), 0, st, a); }
  return hipGetLastError();
}

hipError_t launch_onehot(const int32_t* argmax, int32_t n_batch, int32_t n_recv, int32_t n_send,
                         float* M, hipStream_t st) {
  const int64_t tot = (int64_t)n_batch * n_recv * n_send;
  if (tot == 0) return hipSuccess;
  {
    KernelTimer kt_("k_onehot", st);
    hipLaunchKernelGGL(k_onehot, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, argmax,
                       (int64_t)n_batch * n_recv, n_send, M);
  }
  return hipGetLastError();
}

}  // namespace cma
