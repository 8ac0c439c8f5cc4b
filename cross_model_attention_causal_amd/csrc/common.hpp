// Shared device helpers for the gfx950 kernels: bf16 conversion, MFMA wrappers,
// cross-lane exchange and packed-sequence index math.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cma.h"

namespace cma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 lds_bf16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;    // accelerator complex dies; workgroup i runs on XCD i % 8
constexpr int kBlock = 64;  // block-sparse tile edge (rows and columns)
constexpr int kPanel = 16;  // columns per panel of a stored block
// Element (i, j) of a stored 64x64 block: blocks are kept as four panels of 16
// columns, each panel row-major, so a 16-column slice of consecutive rows is
// contiguous in memory.
__device__ __forceinline__ int blk_off(int i, int j) { return (j >> 4) * (kBlock * kPanel) + i * kPanel + (j & 15); }

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest, ties to even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two fp32 -> packed bf16 pair (lo in the low half), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  const bf16x2 r = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// ------------------------------------------------------------------ MFMA
// 16x16x32 bf16: A[m=l%16][k=8(l/16)+e], B[k=8(l/16)+e][n=l%16], D[m=4(l/16)+v][n=l%16]
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 32x32x16 bf16: A[m=l%32][k=8(l/32)+e], B[k=8(l/32)+e][n=l%32],
//                D[m=8(v/4)+4(l/32)+(v%4)][n=l%32]
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// 16-byte load of 8 bf16 elements [j0, j0+8) of a row that is valid for j < n;
// elements at or beyond n read as zero (and are never touched in memory).
__device__ __forceinline__ u32x4 ldg16_guard(const uint16_t* row, int64_t j0, int64_t n) {
  if (j0 + 8 <= n) return ldg16(row + j0);
  u32x4 r = {0u, 0u, 0u, 0u};
  if (j0 >= n) return r;
  uint16_t t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = (j0 + e < n) ? row[j0 + e] : (uint16_t)0;
  r[0] = t[0] | ((uint32_t)t[1] << 16);
  r[1] = t[2] | ((uint32_t)t[3] << 16);
  r[2] = t[4] | ((uint32_t)t[5] << 16);
  r[3] = t[6] | ((uint32_t)t[7] << 16);
  return r;
}

// As ldg16_guard, for rows that may not be 16-byte aligned.
__device__ __forceinline__ u32x4 ldg16_guard_any(const uint16_t* row, int64_t j0, int64_t n) {
  if (((reinterpret_cast<uintptr_t>(row + j0)) & 15) == 0) return ldg16_guard(row, j0, n);
  uint16_t t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = (j0 + e < n) ? row[j0 + e] : (uint16_t)0;
  u32x4 r;
  r[0] = t[0] | ((uint32_t)t[1] << 16);
  r[1] = t[2] | ((uint32_t)t[3] << 16);
  r[2] = t[4] | ((uint32_t)t[5] << 16);
  r[3] = t[6] | ((uint32_t)t[7] << 16);
  return r;
}

// Buffer descriptor word 3 for raw (unformatted) accesses on gfx9-family chips.
// Accesses at or past num_records bytes read zero and drop their writes.
constexpr int kBufferFlags = 0x00020000;
constexpr uint32_t kBufferOff = 0x80000000u;  // an offset past any descriptor used here
constexpr int kCacheNT = 2;                   // cache-policy bit of a buffer access: non-temporal
constexpr int kWaitVmcnt0 = 0x0f70;           // s_waitcnt immediate: vmcnt(0), other counters free

// ------------------------------------------------------------------ cross-lane
__device__ __forceinline__ float xor_lane(float v, int mask) { return __shfl_xor(v, mask, 64); }

// IEEE 754-2019 maximum: a NaN operand gives NaN. Unlike fmaxf it needs no
// quieting of its operands, and chains of it fuse into v_maximum3_f32.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max and sum of a value over the lane pair (l, l ^ 32), both lanes ending with
// the same bits: one v_permlane32_swap (a vector instruction) instead of an LDS
// permute. The swap of (v, v) leaves lanes 0-31 with (own, partner) and lanes
// 32-63 with (partner, own); max and + are commutative.
__device__ __forceinline__ float pair32_max(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair32_add(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Inclusive prefix sum of a float over the 64 lanes in lane order, on data-parallel
// (DPP) lane moves, no LDS: Hillis-Steele steps of 1, 2, 4 and 8 lanes inside each
// row of 16, then each row's total broadcast into the rows after it (lane 15 into
// rows 1 and 3, lane 31 into rows 2 and 3). A fixed tree, so the result is the same
// on every run. Lanes with no source lane add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_from(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float wave_scan_add(float x) {
  x += dpp_from<0x111, 0xf>(x);  // row_shr:1
  x += dpp_from<0x112, 0xf>(x);  // row_shr:2
  x += dpp_from<0x114, 0xf>(x);  // row_shr:4
  x += dpp_from<0x118, 0xf>(x);  // row_shr:8
  x += dpp_from<0x142, 0xa>(x);  // row_bcast:15
  x += dpp_from<0x143, 0xc>(x);  // row_bcast:31
  return x;
}

// Workgroup barrier that waits for this wave's LDS accesses but, unlike
// __syncthreads, not for its global loads (prefetches stay in flight). The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Point between LDS accesses of different lanes of one wave (one lane writes
// what another reads). The hardware runs a wave's LDS instructions in issue
// order, so only the compiler has to be kept from moving accesses across this
// point or reusing values loaded before it.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ packed sequences
struct Varlen {
  int32_t n_seqs;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* used_q;
  const int32_t* used_k;
  int64_t total_q;
  int64_t total_k;
};

// Read-only kernel input (sequence bounds, head scales): loaded through the
// constant address space, so a wave-uniform address becomes a scalar load. Such
// loads are counted apart from the vector memory queue, so waiting for them does
// not also wait for a kernel's prefetches and stores in flight.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

__device__ __forceinline__ int32_t cu_q_of(const Varlen& v, int s) { return ld_const(v.cu_q + s); }
__device__ __forceinline__ int32_t cu_k_of(const Varlen& v, int s) { return ld_const(v.cu_k + s); }
__device__ __forceinline__ int32_t seq_len_q(const Varlen& v, int s) {
  return v.used_q ? ld_const(v.used_q + s) : cu_q_of(v, s + 1) - cu_q_of(v, s);
}
__device__ __forceinline__ int32_t seq_len_k(const Varlen& v, int s) {
  return v.used_k ? ld_const(v.used_k + s) : cu_k_of(v, s + 1) - cu_k_of(v, s);
}

// Elements of one (head, sequence) map in the given layout.
__device__ __forceinline__ int64_t map_elems(int64_t nq, int64_t nk, bool packed) {
  return packed ? nq * (nk - nq) + nq * (nq + 1) / 2 : nq * nk;
}
// Element offset of row i inside one (head, sequence) map.
__device__ __forceinline__ int64_t map_row_off(int64_t i, int64_t nq, int64_t nk, bool packed) {
  return packed ? i * (nk - nq) + i * (i + 1) / 2 : i * nk;
}
// Offset of sequence s's map inside a head's map area (sum over earlier sequences).
// The per-sequence sums below read the sequence table 16 entries at a time, all
// loads of a group issued before the first use (one uniform branch per group for
// the used-length arrays), so that a batch of many sequences costs a few scalar
// round trips rather than one per sequence.
constexpr int kSeqGroup = 16;
// lengths of sequences t .. t + 15 from the used lengths, else the cu differences
__device__ __forceinline__ void seq_lens16(const int32_t* used, const int32_t* cu, int t, int32_t (&n)[kSeqGroup]) {
  if (used) {
#pragma unroll
    for (int e = 0; e < kSeqGroup; ++e) n[e] = ld_const(used + t + e);
  } else {
    int32_t c[kSeqGroup + 1];
#pragma unroll
    for (int e = 0; e <= kSeqGroup; ++e) c[e] = ld_const(cu + t + e);
#pragma unroll
    for (int e = 0; e < kSeqGroup; ++e) n[e] = c[e + 1] - c[e];
  }
}
__device__ __forceinline__ int64_t map_seq_off(const Varlen& v, int s, bool packed) {
  int64_t off = 0;
  int t = 0;
  for (; t + kSeqGroup <= s; t += kSeqGroup) {
    int32_t nq[kSeqGroup], nk[kSeqGroup];
    seq_lens16(v.used_q, v.cu_q, t, nq);
    seq_lens16(v.used_k, v.cu_k, t, nk);
#pragma unroll
    for (int e = 0; e < kSeqGroup; ++e) off += map_elems(nq[e], nk[e], packed);
  }
  for (; t < s; ++t) off += map_elems(seq_len_q(v, t), seq_len_k(v, t), packed);
  return off;
}
// Block-sparse sequences may be prefill chunks: nq query rows at the end of nk
// keys (bottom-right), with the block grid starting at the sequence's first
// token, so nk - nq must be a multiple of 64; the chunk's block-row r is then
// block-row kb0 + r of the grid and sees key blocks 0 .. kb0 + r. Returns kb0,
// or -1 for a sequence that is not such a chunk (it then has no block-rows).
__device__ __forceinline__ int chunk_kb0(int32_t nq, int32_t nk) {
  return (nk >= nq && ((nk - nq) & (kBlock - 1)) == 0) ? (nk - nq) / kBlock : -1;
}

// Offsets of sequence s in the block-sparse arrays: query block-rows (roff) and
// key blocks (kroff) of earlier sequences, and their block-mass entries (tri_off:
// ceil(nq/64) kb0 + R(R+1)/2 each, the lower triangle for whole prompts).
__device__ __forceinline__ void bsr_offsets(const Varlen& v, int s, int32_t& roff, int32_t& kroff, int64_t& tri_off) {
  int32_t r = 0, kr = 0;
  int64_t t = 0;
  int u = 0;
  auto add = [&](int32_t nq, int32_t nk) {
    const int32_t R = (nq + kBlock - 1) / kBlock, kb = max(chunk_kb0(nq, nk), 0);
    r += R;
    kr += (nk + kBlock - 1) / kBlock;
    t += (int64_t)R * kb + (int64_t)R * (R + 1) / 2;
  };
  for (; u + kSeqGroup <= s; u += kSeqGroup) {
    int32_t nq[kSeqGroup], nk[kSeqGroup];
    seq_lens16(v.used_q, v.cu_q, u, nq);
    seq_lens16(v.used_k, v.cu_k, u, nk);
#pragma unroll
    for (int e = 0; e < kSeqGroup; ++e) add(nq[e], nk[e]);
  }
  for (; u < s; ++u) add(seq_len_q(v, u), seq_len_k(v, u));
  roff = r;
  kroff = kr;
  tri_off = t;
}

// Sequence bounds are trusted to be consistent (nondecreasing cu_seqlens, used
// lengths within the reserved rows); these checks keep every access inside the
// tensors even when they are not.
__device__ __forceinline__ bool seq_ok(const Varlen& v, int s, int32_t nq, int32_t nk) {
  int64_t q0 = cu_q_of(v, s), k0 = cu_k_of(v, s);
  return nq >= 0 && nk >= 0 && nq <= nk && q0 >= 0 && k0 >= 0 && q0 + nq <= v.total_q &&
         k0 + nk <= v.total_k;
}

}  // namespace cma
