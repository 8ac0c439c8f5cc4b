// Microbenchmarks of the chip's ceilings that the kernels are measured against:
// streaming HBM read, write and copy bandwidth, the rate of the vector unit's
// exp2 and fused multiply-add, the sustained rate of the 32x32x16 bf16 matrix
// instruction, and the bandwidth from the L2 caches into the compute units
// (every workgroup re-reads one small buffer, so after the first pass the bytes
// come from each XCD's L2, in the 1 KB-per-instruction shape the fused pass
// uses). Each entry point enqueues one launch on `stream`; the caller times it.
// Not part of the method's path.
#include "common.hpp"

#include "cma_probe.h"

namespace cma {

// grid-stride 16-byte reads of n16 chunks; the xor of what was read goes to
// sink[thread] only if it equals `never` (it does not), so the loads stay.
// CONTIG: workgroup b reads chunks [b * per, (b + 1) * per) in runs of 8 KB (one
// 16-byte chunk per thread, four runs in flight), else a grid-stride loop.
template <bool CONTIG>
__global__ __launch_bounds__(512) void k_probe_read(const u32x4* __restrict__ src, int64_t n16, uint32_t never,
                                                     uint32_t* sink) {
  uint32_t x = 0;
  int64_t i, end, step;
  if (CONTIG) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    i = (int64_t)blockIdx.x * per + threadIdx.x;
    end = min(n16, ((int64_t)blockIdx.x + 1) * per);
    step = blockDim.x;
  } else {
    i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    end = n16;
    step = (int64_t)gridDim.x * blockDim.x;
  }
  for (; i < end; i += 4 * step) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i + u * step < end ? src[i + u * step] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (x == never) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

__global__ __launch_bounds__(512) void k_probe_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                     int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// 16-byte stores of n16 chunks. NT: non-temporal (the cache policy the block
// extraction's stores use), else plain. CONTIG: workgroup b writes chunks
// [b * per, (b + 1) * per) in runs of 8 KB (one chunk per thread), else a
// grid-stride loop over all chunks.
template <bool NT, bool CONTIG>
__global__ __launch_bounds__(512) void k_probe_write(u32x4* __restrict__ dst, int64_t n16) {
  const uint32_t v = threadIdx.x;
  int64_t i, end, step;
  if (CONTIG) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    i = (int64_t)blockIdx.x * per + threadIdx.x;
    end = min(n16, ((int64_t)blockIdx.x + 1) * per);
    step = blockDim.x;
  } else {
    i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    end = n16;
    step = (int64_t)gridDim.x * blockDim.x;
  }
  for (; i < end; i += step) {
    if (NT) __builtin_nontemporal_store(u32x4{v, v, v, v}, dst + i);
    else dst[i] = u32x4{v, v, v, v};
  }
}

// Every lane runs `iters` rounds of 8 independent chains of one vector operation
// (kind 0: exp2, the hardware transcendental; kind 1: fused multiply-add).
template <int KIND>
__global__ __launch_bounds__(256) void k_probe_valu(int iters, float* out) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)(threadIdx.x + i) * 1e-3f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = KIND == 0 ? __builtin_amdgcn_exp2f(x[i]) : fmaf(x[i], 0.999f, 0.5f);
  }
  float r = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) r += x[i];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// Every lane reads 16 bytes per instruction from LDS, 8 reads in flight, lane L
// of a wave at byte 16 L of a 1 KB run (the pattern the kernels' operand reads
// use, free of bank conflicts), `iters` rounds over a 64 KB buffer.
__global__ __launch_bounds__(512) void k_probe_lds(int iters, uint32_t never, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint32_t buf[16384];  // 64 KB
  for (int i = threadIdx.x; i < 16384; i += 512) buf[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t x = 0;
  for (int it = 0; it < iters; ++it) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int run = (it * 8 + u + wave * 8) & 63;  // 64 runs of 1 KB
      v[u] = *reinterpret_cast<const u32x4*>(&buf[run * 256 + 4 * lane]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u][0] ^ v[u][3];
  }
  if (x == never) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

// Every wave runs `iters` rounds of 8 independent 32x32x16 bf16 products.
__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  u32x4 av = {0x3f803f80u ^ (uint32_t)lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  u32x4 bv = {0x3c003c00u, 0x3c003c00u ^ (uint32_t)lane, 0x3c003c00u, 0x3c003c00u};
  f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = mfma32(as_bf16x8(av), as_bf16x8(bv), acc[k]);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[k][v];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Every workgroup reads the same `bytes` (a multiple of 16 KB) `iters` times, one
// 1 KB-per-wave buffer load per instruction, 8 loads in flight per wave.
__global__ __launch_bounds__(512) void k_probe_l2(const uint16_t* __restrict__ buf, int bytes, int iters,
                                                   uint32_t never, uint32_t* sink) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(buf), (short)0, bytes, kBufferFlags);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t x = 0;
  const int per_round = 8 * 1024 * 8;  // 8 waves x 8 loads x 1 KB
  for (int it = 0; it < iters; ++it) {
    for (int off = 0; off < bytes; off += per_round) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, 16u * lane, off + (wave * 8 + u) * 1024, 0);
#pragma unroll
      for (int u = 0; u < 8; ++u) x ^= v[u][0] ^ v[u][3];
    }
  }
  if (x == never) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

}  // namespace cma

using namespace cma;

extern "C" {

int cma_probe_read(const void* src, int64_t bytes, int32_t n_wg, int32_t mode, void* sink, void* stream) {
  if (!src || !sink || bytes < 16 || n_wg < 1 || (mode != 0 && mode != 1) || (reinterpret_cast<uintptr_t>(src) & 15))
    return CMA_EINVAL;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (mode == 0)
    hipLaunchKernelGGL((k_probe_read<false>), dim3(n_wg), dim3(512), 0, st, static_cast<const u32x4*>(src), bytes / 16,
                       0x9e3779b9u, static_cast<uint32_t*>(sink));
  else
    hipLaunchKernelGGL((k_probe_read<true>), dim3(n_wg), dim3(512), 0, st, static_cast<const u32x4*>(src), bytes / 16,
                       0x9e3779b9u, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? CMA_OK : CMA_EHIP;
}

int cma_probe_copy(const void* src, void* dst, int64_t bytes, int32_t n_wg, void* stream) {
  if (!src || !dst || bytes < 16 || n_wg < 1 || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15))
    return CMA_EINVAL;
  hipLaunchKernelGGL(k_probe_copy, dim3(n_wg), dim3(512), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? CMA_OK : CMA_EHIP;
}

int cma_probe_write(void* dst, int64_t bytes, int32_t n_wg, int32_t mode, void* stream) {
  if (!dst || bytes < 16 || n_wg < 1 || mode < 0 || mode > 3 || (reinterpret_cast<uintptr_t>(dst) & 15))
    return CMA_EINVAL;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  u32x4* d = static_cast<u32x4*>(dst);
  const int64_t n16 = bytes / 16;
  switch (mode) {
    case 0: hipLaunchKernelGGL((k_probe_write<false, false>), dim3(n_wg), dim3(512), 0, st, d, n16); break;
    case 1: hipLaunchKernelGGL((k_probe_write<true, false>), dim3(n_wg), dim3(512), 0, st, d, n16); break;
    case 2: hipLaunchKernelGGL((k_probe_write<false, true>), dim3(n_wg), dim3(512), 0, st, d, n16); break;
    default: hipLaunchKernelGGL((k_probe_write<true, true>), dim3(n_wg), dim3(512), 0, st, d, n16); break;
  }
  return hipGetLastError() == hipSuccess ? CMA_OK : CMA_EHIP;
}

int cma_probe_valu(int32_t kind, int32_t n_wg, int32_t iters, float* out, void* stream) {
  if (!out || n_wg < 1 || iters < 1 || (kind != 0 && kind != 1)) return CMA_EINVAL;
  if (kind == 0)
    hipLaunchKernelGGL(k_probe_valu<0>, dim3(n_wg), dim3(256), 0, static_cast<hipStream_t>(stream), iters, out);
  else
    hipLaunchKernelGGL(k_probe_valu<1>, dim3(n_wg), dim3(256), 0, static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? CMA_OK : CMA_EHIP;
}

int cma_probe_mfma(int32_t n_wg, int32_t iters, float* out, void* stream) {
  if (!out || n_wg < 1 || iters < 1) return CMA_EINVAL;
  hipLaunchKernelGGL(k_probe_mfma, dim3(n_wg), dim3(256), 0, static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? CMA_OK : CMA_EHIP;
}

int cma_probe_lds(int32_t n_wg, int32_t iters, void* sink, void* stream) {
  if (!sink || n_wg < 1 || iters < 1) return CMA_EINVAL;
  hipLaunchKernelGGL(k_probe_lds, dim3(n_wg), dim3(512), 0, static_cast<hipStream_t>(stream), iters, 0x9e3779b9u,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? CMA_OK : CMA_EHIP;
}

int cma_probe_l2(const void* buf, int32_t bytes, int32_t iters, int32_t n_wg, void* sink, void* stream) {
  if (!buf || !sink || n_wg < 1 || iters < 1 || bytes < 65536 || bytes % 65536) return CMA_EINVAL;
  hipLaunchKernelGGL(k_probe_l2, dim3(n_wg), dim3(512), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(buf), bytes, iters, 0x9e3779b9u, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? CMA_OK : CMA_EHIP;
}

}  // extern "C"
