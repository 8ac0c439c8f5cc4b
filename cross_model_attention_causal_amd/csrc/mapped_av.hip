// Fused mapped attention x V (MapFlow, approach and storage-and-execution
// sections; IAM Method 4 for decode rows):  O_h = (sum_j M[h, j] A_j) V_h.
//
// Block-sparse source (k_mapped_av_bsr). A workgroup (8 waves) owns 32 query
// rows of one block-row and a group of at most 12 receiver heads. It first
// lists, in LDS, the block columns that any sender kept (ascending) and, per
// column and sender, which stored block holds it. It then walks the key axis in
// 16-key panels (four per 64-key block column) with a software pipeline; in
// step t
//   - the 32 senders' 32 x 16 pieces of panel t + 2 (one contiguous 1 KB run of
//     a stored block's 16-column panel per sender, or zeros for a sender that did
//     not keep the block), loaded into registers in step t - 2, are
//     written to LDS, and those of panel t + 4 are loaded (two register sets,
//     so that every global read has two steps to arrive);
//   - the V operands of panel t + 2 are loaded into a ring of registers;
//   - panel t + 1 is mixed on the matrix cores: D1[h, pos] = sum_j M[h, j]
//     A_j[pos] for 16 positions is a 16x16x32 MFMA with M (split into bf16 high
//     and low parts, so the mix is accurate to ~2^-16) as the A operand and the
//     senders, read with the transposing LDS load so that each lane gets 8
//     senders of one position, as the B operand; the mixed maps B_h go to LDS
//     as bf16;
//   - O += B_h V_h over panel t on 32x32x16 MFMAs, fp32 accumulators in
//     registers; the group's (head, 32-feature tile) products are dealt evenly
//     over the waves.
// One barrier per step. The mixed map never leaves LDS.
//
// Dense source (k_mapped_av_dense): one workgroup per (query row, sequence,
// receiver head) mixes the visible part of the row into LDS (only the nonzero
// mixing weights are read, so a one-hot M reads one sender row) and streams V
// with 16-byte loads. Used for decode rows and small dense problems.
#include <type_traits>

#include "kernels.hpp"

namespace cma {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsPerWg = 12;      // receiver heads per workgroup (M rows 12..15 of the mix are unused)
constexpr int kRowsPerWg = 32;
constexpr int kKeysPerStep = 16;     // one panel
constexpr int kSend = 32;            // senders per workgroup (n_send <= 32)
constexpr int kSendStride = 544;     // bf16 per staged sender: 32 rows x 16 keys + 32 pad
constexpr int kStageElems = kSend * kSendStride;
constexpr int kStages = 2;           // sender stages: panel t + 1 read while panel t + 2 is written
constexpr int kBH = 520;             // bf16 per head of a mixed panel: 32 rows x 16 keys + 8 pad
constexpr int kBBuf = 16 * kBH;      // one mixed panel, 16 head slots (the mix's M rows)
constexpr int kMaxCols = 256;        // block columns per sequence (16384 tokens)
constexpr uint16_t kNoBlock = 0xffff;

// V in the fused kernel's operand order ("tiled"): for head h and 64-key block b
// of the block grid (sequence s's blocks start at its block-row offset, as in
// the block-sparse maps), 16 KB hold, for panel ks (16 keys) and feature tile dt
// (32 features), 64 lanes x 8 keys: lane L, element e is
//   V[key 64c + 16ks + 8(L / 32) + e][feature 32dt + L % 32],
// zero past the sequence end. One 16-byte load per lane reads a whole
// contiguous 1 KB MFMA operand, and the four operands of a panel are adjacent.
__device__ __forceinline__ int vtile_pos(int ks, int dt, int lane) { return ((ks * 4 + dt) * 64 + lane) * 8; }

// grid (key blocks of the longest sequence, n_seqs, n_v), 256 threads: one 64-key
// block of one V head, written to the sequence's tiled blocks (starting at its
// key-block offset) or, with a page table, to the page the table names.
template <bool KEY_MAJOR>
__global__ __launch_bounds__(256) void k_tile_v(const uint16_t* __restrict__ v, uint16_t* __restrict__ vtile,
                                                Varlen vl, int32_t n_key_blocks, const int32_t* __restrict__ pages,
                                                int32_t page_stride, int32_t n_pages) {
  constexpr int D = 128;
  __shared__ uint16_t tile[64][D + 8];
  const int c = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const int32_t n = seq_len_k(vl, s);
  const int64_t kbase = cu_k_of(vl, s);
  if (n < 0 || kbase < 0 || kbase + n > vl.total_k || 64 * c >= n) return;
  uint16_t* dst;
  if (pages) {
    const int32_t pg = ld_const(pages + (int64_t)s * page_stride + c);
    if (pg < 0 || pg >= n_pages) return;
    dst = vtile + ((int64_t)h * n_pages + pg) * (64 * D);
  } else {
    int32_t roff, kroff;
    int64_t tri;
    bsr_offsets(vl, s, roff, kroff, tri);
    dst = vtile + ((int64_t)h * n_key_blocks + kroff + c) * (64 * D);
  }
  const int64_t k0 = kbase + 64 * c;
  const int valid = min(64, n - 64 * c);
  if (KEY_MAJOR) {
    // rows of 64 keys per feature: 8 lanes x 16 B per feature row
    for (int x = threadIdx.x; x < D * 8; x += 256) {
      const int f = x >> 3, k8 = 8 * (x & 7);
      const uint16_t* src = v + ((int64_t)h * D + f) * vl.total_k + k0 + k8;
      for (int e = 0; e < 8; ++e) tile[k8 + e][f] = (k8 + e < valid) ? src[e] : (uint16_t)0;
    }
  } else {
    // 64 contiguous key rows of 256 B
    for (int x = threadIdx.x; x < 64 * (D / 8); x += 256) {
      const int key = x / (D / 8), f8 = 8 * (x % (D / 8));
      u32x4 w = {0u, 0u, 0u, 0u};
      if (key < valid) w = ldg16(v + ((int64_t)h * vl.total_k + k0 + key) * D + f8);
      *reinterpret_cast<u32x4*>(&tile[key][f8]) = w;
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < 64 * D / 8; x += 256) {
    // x = (ks * 4 + dt) * 64 + lane
    const int lane = x & 63, kd = x >> 6, dt = kd & 3, ks = kd >> 2;
    const int key0 = 16 * ks + 8 * (lane >> 5), f = 32 * dt + (lane & 31);
    uint32_t w[4];
    for (int e = 0; e < 4; ++e) w[e] = tile[key0 + 2 * e][f] | ((uint32_t)tile[key0 + 2 * e + 1][f] << 16);
    *reinterpret_cast<u32x4*>(dst + (int64_t)x * 8) = u32x4{w[0], w[1], w[2], w[3]};
  }
}


// Work items are (sequence, pair of block-rows, row half, head group). Pair pr
// of a sequence with R block-rows holds rows R - 1 - pr and pr: the long row is
// swept with its key columns ascending, then the short row with its columns
// descending. Every pair then covers R + 1 columns, so the workgroups of a
// launch wave start together and stay in step, and at any time they all work on
// one of two columns (tau and R + 1 - tau): each V tile and each sender column is
// fetched once per XCD and then served from its L2 to all of them. Items of one
// (sequence, pair) "unit" share sender rows (head groups) and V tiles (row
// halves) and sit on the same XCD: the hardware deals workgroup ids round-robin
// over the 8 XCDs, so id i runs on XCD i % 8 and is that XCD's (i / 8)-th
// workgroup, and unit u goes to XCD u % 8; units are numbered pair-major with
// the sequences interleaved, so with up to 8 sequences an XCD keeps to the same
// sequences.
__device__ __forceinline__ bool decode_item(int id, int n_seqs, int n_pairs, int n_hg, int& s, int& pr, int& rh,
                                            int& hg) {
  const int per_unit = 2 * n_hg;
  const int xcd = id % kXcds, m = id / kXcds;
  const int k = m / per_unit, item = m % per_unit;
  const int u = kXcds * k + xcd;
  if (u >= n_seqs * n_pairs) return false;
  pr = u / n_seqs;
  s = u % n_seqs;
  rh = item & 1;
  hg = item >> 1;
  return true;
}

// LDS address of a shared-memory object, as the asm below takes it.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const T*)p);
}

// LDS accesses of the pipelined loop are written in asm, each statement issuing
// its accesses and (for reads) waiting for them, so the LDS traffic of a step is
// explicit. An asm statement that issues several reads from one address
// register marks its outputs early-clobber ("=&v"): otherwise the compiler may
// give the first read's destination the address register, and a read that
// returns before the next one issues would overwrite the address the later
// reads use.
__device__ __forceinline__ int lds_u16(const uint16_t* p) {
  uint32_t v;
  asm volatile("ds_read_u16 %0, %1\n"
               "s_waitcnt lgkmcnt(0)"
               : "=v"(v)
               : "v"(lds_addr(p))
               : "memory");
  return __builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ int lds_i32(const int* p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n"
               "s_waitcnt lgkmcnt(0)"
               : "=v"(v)
               : "v"(lds_addr(p))
               : "memory");
  return __builtin_amdgcn_readfirstlane((int)v);
}

// grid (8 * ceil(units / 8) * 2 * n_hg), kThreads threads.
__global__ __launch_bounds__(kThreads) void k_mapped_av_bsr(MappedAvArgs a, int n_pairs, int n_hg, int hpg) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(16))) uint16_t sbuf[kStages * kStageElems];
  __shared__ __attribute__((aligned(16))) uint16_t bbuf[2 * kBBuf];
  __shared__ uint16_t tbl[kMaxCols * kSend];  // block index - sender's first block, or kNoBlock
  __shared__ uint16_t ucol[kMaxCols];         // kept columns (any sender), ascending
  __shared__ int upage[kMaxCols];             // V block (tiled or paged) of each kept column
  __shared__ int sbeg[kSend];
  __shared__ int nu_s;
  __shared__ uint8_t anyc[kMaxCols];

  int s, pr, rh, hg;
  if (!decode_item(blockIdx.x, a.vl.n_seqs, n_pairs, n_hg, s, pr, rh, hg)) return;
  // n query rows at the end of nk keys (a prefill chunk; n = nk for a whole
  // prompt): block-row r of the queries is block-row kb0 + r of the sequence
  const int32_t n = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
  const int kb0 = chunk_kb0(n, nk);
  if (!seq_ok(a.vl, s, n, nk) || kb0 < 0) return;
  const int r_long = (n + kBlock - 1) / kBlock - 1 - pr;  // swept first, columns ascending
  if (r_long < pr) return;                                 // past this sequence's pairs
  const int n_pass = r_long > pr ? 2 : 1;                  // then row pr, columns descending
  // the wave index is uniform: keep it (and what is derived from it) in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  int32_t roff, kroff;
  int64_t tri;
  bsr_offsets(a.vl, s, roff, kroff, tri);
  const bool paged = a.v_pages != nullptr;

  // Block table of block-row r (key blocks 0 .. kb0 + r): tbl[c][j] = kept block
  // of sender j at column c, ucol = the union of kept columns in ascending order
  // (nu_s of them), upage = the V block of each, sbeg[j] = sender j's first block
  // of the row.
  auto build_table = [&](int r) __attribute__((always_inline)) {
    const int ra = kb0 + r;
    __syncthreads();  // the previous row's readers are done with these arrays
    for (int x = tid; x < (ra + 1) * kSend; x += kThreads) tbl[x] = kNoBlock;
    for (int c = tid; c <= ra; c += kThreads) anyc[c] = 0;
    if (tid < kSend) sbeg[tid] = (tid < a.n_send) ? a.row_ptr[(int64_t)(a.send0 + tid) * a.n_block_rows + roff + r] : 0;
    __syncthreads();
    {
      constexpr int kPer = kThreads / kSend;  // threads per sender
      const int j = tid / kPer, e0 = tid % kPer;
      if (j < a.n_send) {
        const int64_t g = (int64_t)(a.send0 + j) * a.n_block_rows + roff + r;
        const int beg = a.row_ptr[g], end = a.row_end ? a.row_end[g] : a.row_ptr[g + 1];
        for (int e = beg + e0; e < end; e += kPer) {
          const int c = a.col_idx[e];
          if (c >= 0 && c <= ra && e - beg < (int)kNoBlock) {
            tbl[c * kSend + j] = (uint16_t)(e - beg);
            anyc[c] = 1;
          }
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      int base = 0;
      for (int c0 = 0; c0 <= ra; c0 += 64) {
        const int c = c0 + lane;
        const bool f = c <= ra && anyc[c];
        const uint64_t m = __ballot(f);
        if (f) ucol[base + __popcll(m & ((1ull << lane) - 1ull))] = (uint16_t)c;
        base += __popcll(m);
      }
      if (lane == 0) nu_s = base;
    }
    __syncthreads();
    for (int x = tid; x < nu_s; x += kThreads) {
      const int c = ucol[x];
      // a page outside the pool (a broken table) is clamped into it: memory-safe
      upage[x] = paged ? min(max(a.v_pages[(int64_t)s * a.v_page_stride + c], 0), a.v_n_pages - 1) : c;
    }
    __syncthreads();
  };

  // Head group hg holds heads hg * hpg .. + hpg - 1 (hpg <= 12: the receiver
  // heads split evenly over the groups, so that the groups of a block-row take
  // the same time and read the shared sender rows together).
  const int h_lo = hg * hpg, heads_here = min(hpg, a.n_recv - h_lo);
  // ---- mixing weights, A operand of 16x16x32: lane (p, q) holds M[h_lo + p][8q + e]
  bf16x8 mhi, mlo;
  {
    const int p = lane & 15, q = lane >> 4;
    const int h = h_lo + p;
    const float* Ms = a.M + (int64_t)s * a.M_stride;
    u32x4 hi, lo;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      float xh[2], xl[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = 8 * q + 2 * e2 + u;
        const float x = (p < heads_here && j < a.n_send) ? Ms[(int64_t)h * a.m_ld + a.send0 + j] : 0.0f;
        xh[u] = bf2f(f2bf(x));
        xl[u] = x - xh[u];
      }
      hi[e2] = pack2bf(xh[0], xh[1]);
      lo[e2] = pack2bf(xl[0], xl[1]);
    }
    mhi = as_bf16x8(hi);
    mlo = as_bf16x8(lo);
  }
  // per block-row: start of this wave's senders (j = wave + 8u) in the
  // block-sparse arrays, and the row's panel count and sweep direction
  int sb[kSend / kWaves];
  int nu = 0, T = 0;
  bool rev = false;
  // k-th kept column of the row in sweep order
  auto col_at = [&](int k) __attribute__((always_inline)) { return lds_u16(&ucol[rev ? nu - 1 - k : k]); };
  // its V block (offset in 64-key blocks from the V descriptor's base)
  auto page_at = [&](int k) __attribute__((always_inline)) { return lds_i32(&upage[rev ? nu - 1 - k : k]); };
  const int q = lane >> 4, p = lane & 15, e4 = (lane >> 2) & 3, cc4 = lane & 3;
  const int n32 = lane & 31, q2 = lane >> 5;
  // Sources of this wave's senders for one block column: the stored block's rows
  // of this row half, or, for a sender that did not keep the block, a descriptor
  // of no bytes (its loads return zeros without a memory access: dropping these
  // reads shortened the pass by 5 %, the per-CU memory path being its bound).
  // Global reads go through buffer descriptors: the base and the per-step offset
  // are scalar, the per-lane offset is one register, and a read past the
  // descriptor's size returns zeros instead of touching memory.
  struct SendSrc {
    __amdgpu_buffer_rsrc_t r[kSend / kWaves];
    int step[kSend / kWaves];  // bytes per panel: 2 KB, or 0 for a dropped block
  };
  auto col_src = [&](int c, SendSrc& ss) __attribute__((always_inline)) {
    // tbl entries of senders wave, wave + 8, wave + 16, wave + 24 are 16 B apart
    uint32_t t4[4];
    asm volatile("ds_read_u16 %0, %4\n"
                 "ds_read_u16 %1, %4 offset:16\n"
                 "ds_read_u16 %2, %4 offset:32\n"
                 "ds_read_u16 %3, %4 offset:48\n"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(t4[0]), "=&v"(t4[1]), "=&v"(t4[2]), "=&v"(t4[3])
                 : "v"(lds_addr(&tbl[c * kSend + wave]))
                 : "memory");
    static_assert(kSend / kWaves == 4 && kWaves * 2 == 16, "the offsets above assume this geometry");
#pragma unroll
    for (int u = 0; u < kSend / kWaves; ++u) {
      const int bi = __builtin_amdgcn_readfirstlane((int)t4[u]);
      const bool kept = bi != kNoBlock;
      // this row half's rows of the stored block: 3 panels x 2 KB + 1 KB reachable
      const uint16_t* base =
          kept ? a.vals + (int64_t)(sb[u] + bi) * (kBlock * kBlock) + (kRowsPerWg * rh) * kPanel : a.vals;
      ss.r[u] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0,
                                                  kept ? 2 * (kBlock * kBlock - kRowsPerWg * rh * kPanel) : 0,
                                                  kBufferFlags);
      ss.step[u] = kept ? 2 * kBlock * kPanel : 0;
    }
  };
  // Panel jq (16 keys) of the column: each sender's 1 KB piece is loaded into
  // registers, 16 B per lane (lane L holds row L / 2, half L % 2), and written
  // to a stage buffer. Senders j with bit 3 set store row r at row position
  // r ^ 1: the transposing reads of senders j and j + 8 then fall in different
  // LDS banks.
  const uint32_t loff0 = 16u * lane, loff1 = 16u * (lane ^ 2);
  // Non-temporal: a stored block is read by the two head groups' workgroups and then
  // not again (2-3 % faster than the default policy).
  auto load_stage = [&](const SendSrc& ss, int jq, u32x4 (&S)[kSend / kWaves]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kSend / kWaves; ++u)  // sender wave + 8u: (j >> 3) & 1 == u & 1
      S[u] = __builtin_amdgcn_raw_buffer_load_b128(ss.r[u], (u & 1) ? loff1 : loff0, jq * ss.step[u], kCacheNT);
  };
  static_assert(kSend / kWaves == 4 && kWaves * kSendStride * 2 == 8704, "the offsets below assume this geometry");
  auto store_stage = [&](const u32x4 (&S)[kSend / kWaves], int b) __attribute__((always_inline)) {
    asm volatile(
        "ds_write_b128 %0, %1\n"
        "ds_write_b128 %0, %2 offset:8704\n"
        "ds_write_b128 %0, %3 offset:17408\n"
        "ds_write_b128 %0, %4 offset:26112" ::"v"(lds_addr(&sbuf[b * kStageElems + wave * kSendStride]) + 16u * lane),
        "v"(S[0]), "v"(S[1]), "v"(S[2]), "v"(S[3])
        : "memory");
  };
  // LDS reads of one step, in one asm statement with one wait: the eight
  // transposing reads of the panel to mix (lane (p, q) gets senders 8q .. 8q + 7
  // at key p of rows wave + 8u; senders 8q + e4 (+ 4), row wave + 8u at row
  // position (wave ^ (q & 1)) + 8u) and the two mixed-map operands of the
  // products.
  static_assert(kRowsPerWg / kWaves == 4 && kKeysPerStep * kWaves * 2 == 256 && kSendStride * 8 == 4352,
                "the offsets below assume this stage geometry");
  const uint32_t tr_lane = 2u * ((8 * q + e4) * kSendStride + (wave ^ (q & 1)) * kKeysPerStep + 4 * cc4);
  auto read_mix_src = [&](int b, u32x2 (&tr)[8]) __attribute__((always_inline)) {
    const uint32_t a0 = lds_addr(&sbuf[b * kStageElems]) + tr_lane;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n"
        "ds_read_b64_tr_b16 %1, %8 offset:4352\n"
        "ds_read_b64_tr_b16 %2, %8 offset:256\n"
        "ds_read_b64_tr_b16 %3, %8 offset:4608\n"
        "ds_read_b64_tr_b16 %4, %8 offset:512\n"
        "ds_read_b64_tr_b16 %5, %8 offset:4864\n"
        "ds_read_b64_tr_b16 %6, %8 offset:768\n"
        "ds_read_b64_tr_b16 %7, %8 offset:5120\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(tr[0]), "=&v"(tr[1]), "=&v"(tr[2]), "=&v"(tr[3]), "=&v"(tr[4]), "=&v"(tr[5]), "=&v"(tr[6]),
          "=&v"(tr[7])
        : "v"(a0)
        : "memory");
  };
  auto read_step = [&](int b, u32x2 (&tr)[8], uint32_t oa_addr, uint32_t ob_addr, u32x4& oa, u32x4& ob)
                       __attribute__((always_inline)) {
    const uint32_t a0 = lds_addr(&sbuf[b * kStageElems]) + tr_lane;
    asm volatile(
        "ds_read_b128 %8, %10\n"
        "ds_read_b128 %9, %11\n"
        "ds_read_b64_tr_b16 %0, %12\n"
        "ds_read_b64_tr_b16 %1, %12 offset:4352\n"
        "ds_read_b64_tr_b16 %2, %12 offset:256\n"
        "ds_read_b64_tr_b16 %3, %12 offset:4608\n"
        "ds_read_b64_tr_b16 %4, %12 offset:512\n"
        "ds_read_b64_tr_b16 %5, %12 offset:4864\n"
        "ds_read_b64_tr_b16 %6, %12 offset:768\n"
        "ds_read_b64_tr_b16 %7, %12 offset:5120\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(tr[0]), "=&v"(tr[1]), "=&v"(tr[2]), "=&v"(tr[3]), "=&v"(tr[4]), "=&v"(tr[5]), "=&v"(tr[6]),
          "=&v"(tr[7]), "=&v"(oa), "=&v"(ob)
        : "v"(oa_addr), "v"(ob_addr), "v"(a0)
        : "memory");
  };
  // Mix on 16x16x32 MFMAs with the senders as the A operand and M as the B
  // operand: D[key 4q + v][head p] for row wave + 8u lands in lane (p, q), so a
  // lane holds four consecutive keys of one head and writes them as one 8-byte
  // store to bbuf[bb * kBBuf + p * kBH + 16 row + 4q] (head slot, row, key).
  // With the head stride of 1040 B the 64 lanes of a store hit distinct banks.
  const uint32_t mix_lane = 2u * (p * kBH + wave * kKeysPerStep + 4 * q);
  auto mix_store = [&](int bb, const u32x2 (&tr)[8]) __attribute__((always_inline)) {
    u32x2 w[4];
#pragma unroll
    for (int u = 0; u < kRowsPerWg / kWaves; ++u) {
      const u32x4 av = {tr[2 * u][0], tr[2 * u][1], tr[2 * u + 1][0], tr[2 * u + 1][1]};
      f32x4 d = mfma16(as_bf16x8(av), mhi, f32x4{0.f, 0.f, 0.f, 0.f});
      d = mfma16(as_bf16x8(av), mlo, d);
      w[u] = u32x2{pack2bf(d[0], d[1]), pack2bf(d[2], d[3])};
    }
    // rows wave + 8u are 8 x 32 B = 256 B apart
    asm volatile(
        "ds_write_b64 %0, %1\n"
        "ds_write_b64 %0, %2 offset:256\n"
        "ds_write_b64 %0, %3 offset:512\n"
        "ds_write_b64 %0, %4 offset:768" ::"v"(lds_addr(&bbuf[bb * kBBuf]) + mix_lane),
        "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3])
        : "memory");
  };

  // The group's products are items (head slot, feature tile dt), 4 per head,
  // dealt NI to a wave with a fixed shape: items k < NA use head slot sA (tiles
  // dA + k), the rest head slot sB (tiles dB + k - NA).
  //   NI = 6 (up to 12 heads): sA = wave (all four tiles), sB = 8 + wave / 2
  //                            (tiles 2 (wave % 2), + 1)
  //   NI = 4 (up to 8 heads):  sA = wave (all four tiles)
  //   NI = 2 (up to 4 heads):  sA = wave / 2 (tiles 2 (wave % 2), + 1)
  // Slots past the group's heads run the same branch-free schedule on a V
  // descriptor of no bytes (their loads return zeros without a memory access)
  // and are not stored.
  auto run = [&](auto ni) __attribute__((always_inline)) {
    constexpr int NI = decltype(ni)::value;
    constexpr int NA = NI == 2 ? 2 : 4;
    const int w = __builtin_amdgcn_readfirstlane(wave);
    const int sA = NI == 2 ? (w >> 1) : w, dA = NI == 2 ? 2 * (w & 1) : 0;
    const int sB = NI == 6 ? 8 + (w >> 1) : sA, dB = NI == 6 ? 2 * (w & 1) : 0;
    f32x16 acc[NI];
    // V of slots sA and sB (clamped to the group): this sequence's tiled key
    // blocks, or the V head's whole page pool (the column's page is the offset)
    const int v_bytes = (paged ? a.v_n_pages : (nk + kBlock - 1) / kBlock) * (kBlock * D * 2);
    auto v_base = [&](int slot) __attribute__((always_inline)) {
      const int64_t g = (h_lo + min(slot, heads_here - 1)) / a.v_group;
      return const_cast<uint16_t*>(a.vt + (paged ? g * a.v_n_pages : g * a.n_key_blocks + kroff) * (kBlock * D));
    };
    const __amdgpu_buffer_rsrc_t vA =
        __builtin_amdgcn_make_buffer_rsrc(v_base(sA), (short)0, sA < heads_here ? v_bytes : 0, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vB =
        __builtin_amdgcn_make_buffer_rsrc(v_base(sB), (short)0, sB < heads_here ? v_bytes : 0, kBufferFlags);
    // mixed-map operands of slots sA and sB: lane (row n32, half q2) holds keys
    // 8 q2 .. + 7, one contiguous 1 KB read each
    const uint32_t oA_lane = 2u * (sA * kBH + n32 * kKeysPerStep + 8 * q2);
    const uint32_t oB_lane = 2u * (sB * kBH + n32 * kKeysPerStep + 8 * q2);
    SendSrc dsrc;   // sources of the column being copied
    int v_off = 0;  // tiled-V offset of the column being loaded
    u32x4 vr[2][NI];
    const uint32_t vlane = 16u * lane;
    auto load_v = [&](int jq, u32x4 (&dst)[NI]) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int soff = 2 * (v_off + (k < NA ? vtile_pos(jq, dA + k, 0) : vtile_pos(jq, dB + k - NA, 0)));
        dst[k] = __builtin_amdgcn_raw_buffer_load_b128(k < NA ? vA : vB, vlane, soff, 0);
      }
    };
    // Mix the panel in stage b into mixed buffer bbm (when do_mix), and
    // O += B V over the mixed panel in buffer bba with V operands v.
    auto compute = [&](int b, int bbm, bool do_mix, int bba, const u32x4 (&v)[NI]) __attribute__((always_inline)) {
      u32x2 tr[8];
      u32x4 oa, ob;
      const uint32_t ob0 = lds_addr(&bbuf[bba * kBBuf]);
      if (do_mix) {
        read_step(b, tr, ob0 + oA_lane, ob0 + oB_lane, oa, ob);
      } else {
        asm volatile("ds_read_b128 %0, %2\n"
                     "ds_read_b128 %1, %3\n"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(oa), "=&v"(ob)
                     : "v"(ob0 + oA_lane), "v"(ob0 + oB_lane)
                     : "memory");
      }
#pragma unroll
      for (int k = 0; k < NI; ++k) acc[k] = mfma32(as_bf16x8(k < NA ? oa : ob), as_bf16x8(v[k]), acc[k]);
      if (do_mix) mix_store(bbm, tr);
    };

    u32x4 S[2][kSend / kWaves];  // sender pieces of the next two panels to stage

    // Step t: write panel t + 2 (in S[t % 2] since step t - 2) to stage t % 2
    // (panel t's, mixed in step t - 1), load panel t + 4 into S[t % 2], mix
    // panel t + 1 (stage (t + 1) % 2) into mixed buffer (t + 1) % 2, multiply
    // panel t (mixed buffer t % 2) with V slot t % 2, then load V of panel t + 2
    // into that slot. The compiler places the waits for the loaded registers
    // itself; in the main loop a step waits only for loads issued two steps
    // before it (the two later steps' loads stay in flight), because the
    // prologue issues its loads in the loop's order.
    //
    // Main loop: 4 steps per trip, all full (t + 4 < T), with the column changes
    // at fixed steps (panel t + 4 starts a column when t % 4 == 0, panel t + 2
    // when t % 4 == 2).
    auto step_main = [&](int t0, auto ic) __attribute__((always_inline)) {
      constexpr int I = decltype(ic)::value;
      const int t = t0 + I;
      store_stage(S[I & 1], I & 1);
      if constexpr (I == 0) col_src(col_at((t + 4) >> 2), dsrc);
      load_stage(dsrc, I, S[I & 1]);
      compute((I + 1) & 1, (I + 1) & 1, true, I & 1, vr[I & 1]);
      if constexpr (I == 2) v_off = page_at((t + 2) >> 2) * (kBlock * D);
      load_v((I + 2) & 3, vr[I & 1]);
      barrier_lds();
    };
    // The last steps (at most 7): the same work under run-time tests.
    auto step_tail = [&](int t, auto ic) __attribute__((always_inline)) {
      constexpr int I = decltype(ic)::value;  // t % 4 == I
      if (t + 2 < T) store_stage(S[I & 1], I & 1);
      if (t + 4 < T) {
        if (I == 0) col_src(col_at((t + 4) >> 2), dsrc);
        load_stage(dsrc, I, S[I & 1]);
      }
      compute((I + 1) & 1, (I + 1) & 1, t + 1 < T, I & 1, vr[I & 1]);
      if (t + 2 < T) {
        if (I == 2) v_off = page_at((t + 2) >> 2) * (kBlock * D);
        load_v((I + 2) & 3, vr[I & 1]);
      }
      barrier_lds();
    };

    for (int pass = 0; pass < n_pass; ++pass) {
    const int r = pass ? pr : r_long;
    if (64 * r + kRowsPerWg * rh >= n) continue;  // this row half lies past the sequence end
    build_table(r);
    rev = pass == 1;
#pragma unroll
    for (int u = 0; u < kSend / kWaves; ++u) sb[u] = __builtin_amdgcn_readfirstlane(sbeg[wave + kWaves * u]);
    nu = __builtin_amdgcn_readfirstlane(nu_s);
    T = 4 * nu;  // panels
    const int row_base = 64 * r + kRowsPerWg * rh;
#pragma unroll
    for (int k = 0; k < NI; ++k) acc[k] = f32x16{};
    if (T > 0) {
      // prologue (T >= 4, one column at least): panels 0 and 1 staged, panel 0
      // mixed, panels 2 and 3 in S[0] and S[1], V of panels 0 and 1 loaded
      col_src(col_at(0), dsrc);
      v_off = page_at(0) * (kBlock * D);
      load_stage(dsrc, 0, S[0]);
      load_stage(dsrc, 1, S[1]);
      store_stage(S[0], 0);
      store_stage(S[1], 1);
      barrier_lds();
      u32x2 tr[8];
      read_mix_src(0, tr);
      mix_store(0, tr);
      // the loop's loads in its own order (sender panel, V panel, sender panel,
      // V panel), so that the waits the compiler places at the loop head are
      // the loop's own
      load_stage(dsrc, 2, S[0]);
      __builtin_amdgcn_sched_barrier(0);
      load_v(0, vr[0]);
      __builtin_amdgcn_sched_barrier(0);
      load_stage(dsrc, 3, S[1]);
      __builtin_amdgcn_sched_barrier(0);
      load_v(1, vr[1]);
      barrier_lds();
      int t = 0;
      for (; t + 7 < T; t += 4) {
        step_main(t, std::integral_constant<int, 0>{});
        step_main(t, std::integral_constant<int, 1>{});
        step_main(t, std::integral_constant<int, 2>{});
        step_main(t, std::integral_constant<int, 3>{});
      }
      for (; t < T; t += 4) {  // t % 4 == 0 here
        step_tail(t, std::integral_constant<int, 0>{});
        if (t + 1 < T) step_tail(t + 1, std::integral_constant<int, 1>{});
        if (t + 2 < T) step_tail(t + 2, std::integral_constant<int, 2>{});
        if (t + 3 < T) step_tail(t + 3, std::integral_constant<int, 3>{});
      }
    }
    // epilogue: D[m = row][n = feature]: row = 8(v/4) + 4 q2 + (v%4), feature = 32 dt + n32
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int slot = k < NA ? sA : sB, dt = k < NA ? dA + k : dB + k - NA;
      if (slot >= heads_here) continue;
      const int h = h_lo + slot;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = row_base + 8 * (v >> 2) + 4 * q2 + (v & 3);
        if (row >= n) continue;
        const int64_t o = ((int64_t)h * a.vl.total_q + cu_q_of(a.vl, s) + row) * D + 32 * dt + n32;
        if (a.out_bf16) {
          uint16_t* po = reinterpret_cast<uint16_t*>(a.out) + o;
          *po = f2bf(a.accum ? bf2f(*po) + acc[k][v] : acc[k][v]);
        } else {
          float* po = reinterpret_cast<float*>(a.out) + o;
          *po = a.accum ? *po + acc[k][v] : acc[k][v];
        }
      }
    }
    }  // pass
  };
  if (heads_here > 8) run(std::integral_constant<int, 6>{});
  else if (heads_here > 4) run(std::integral_constant<int, 4>{});
  else run(std::integral_constant<int, 2>{});
}

// ------------------------------------------------------------ indexed source
// One sender per receiver head, the head map of IAM Method 4 (the argmax of the
// cosine): O_h = A_{j(h)} V_h. Nothing is mixed. A workgroup owns one receiver
// head and a group of 8 consecutive block-rows of one sequence, one row per
// wave, and sweeps the union of the columns that the head's sender kept in those
// rows. The V block of each column (16 KB in the tiled operand order) is staged
// in LDS once for the 8 rows, so V crosses L2 -> CU once per 8 block-rows
// instead of once per row. A stored block's 16-key panel already holds, for 32
// rows, the A operand of a 32x32x16 MFMA as one contiguous 1 KB run, which the
// wave reads straight into registers three panels ahead (a ring of four sets);
// the V operands come from the stage. Per panel a wave issues 2 global and 4
// LDS reads and 8 MFMAs; a row that did not keep a column skips its products.
//
// Work items are (sequence, pair of row groups, head). Block-rows in the upper
// half of a sequence (2r >= R - 1 for R rows) are swept with their columns
// ascending and the lower ones descending, as the general pass sweeps them, so
// that with a one-hot M both passes add the same terms in the same order (the
// results are bit-identical). Item p takes the upper group of rows R - 8p - 8 ..
// R - 8p - 1 (not below the middle), then the lower group 8p .. 8p + 7 (not
// above it): every item of a sequence covers about R + 8 columns. The heads of a
// sequence are taken in the order of their senders and dealt to XCDs in runs
// (XCD x takes heads x * hpx .. + hpx - 1 of every item), so that heads sharing a
// sender read its blocks from one L2, and each head's V stays in one L2.

// Receiver heads of each sequence ordered by sender (ties by head; heads whose
// sender index is out of range last). grid (n_seqs), 256 threads.
__global__ __launch_bounds__(256) void k_idx_order(MappedAvArgs a) {
  __shared__ int32_t key[256];
  const int s = blockIdx.x, h = threadIdx.x, H = a.n_recv;
  if (h < H) {
    const int j = a.sender[(int64_t)s * a.sender_stride + h];
    key[h] = (j >= 0 && j < a.n_send ? j : a.n_send) * 256 + h;
  }
  __syncthreads();
  if (h < H) {
    const int kh = key[h];
    int rank = 0;
    for (int x = 0; x < H; ++x) rank += key[x] < kh;
    a.plan_order[(int64_t)s * H + rank] = h;
  }
}

constexpr int kIdxRows = 8;  // block-rows per workgroup of the indexed pass (one per wave)

// Block-row offsets of the sequences and the work-item table. One workgroup.
constexpr int kPlanThreads = 1024;
__global__ __launch_bounds__(kPlanThreads) void k_idx_plan(MappedAvArgs a) {
  __shared__ int64_t wsum[kPlanThreads / 64][3];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int64_t x = t; x < a.plan_cap; x += kPlanThreads) a.plan_pairs[x] = -1;
  // exclusive scans of block-rows and pairs over the sequences, in chunks of
  // consecutive sequences per thread
  const int ns = a.vl.n_seqs;
  const int chunk = (ns + kPlanThreads - 1) / kPlanThreads;
  const int s0 = min(ns, t * chunk), s1 = min(ns, s0 + chunk);
  // block-rows (every sequence's, as the block-sparse layout counts them), key
  // blocks, and work pairs (sequences that are whole prompts or valid chunks)
  auto counts = [&](int s, int& nrb, int& nkb, int& np) {
    const int32_t n = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
    nrb = (max(n, 0) + kBlock - 1) / kBlock;
    nkb = (max(nk, 0) + kBlock - 1) / kBlock;
    // items: groups of kIdxRows of the upper ceil(nrb / 2) block-rows (see k_mapped_av_idx)
    np = seq_ok(a.vl, s, n, nk) && chunk_kb0(n, nk) >= 0 ? (nrb - nrb / 2 + kIdxRows - 1) / kIdxRows : 0;
  };
  int64_t rows = 0, kblk = 0, pairs = 0;
  for (int s = s0; s < s1; ++s) {
    int nrb, nkb, np;
    counts(s, nrb, nkb, np);
    rows += nrb;
    kblk += nkb;
    pairs += np;
  }
  int64_t pr = rows, pk = kblk, pp = pairs;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t yr = __shfl_up(pr, off, 64), yk = __shfl_up(pk, off, 64), yp = __shfl_up(pp, off, 64);
    if (lane >= off) {
      pr += yr;
      pk += yk;
      pp += yp;
    }
  }
  if (lane == 63) {
    wsum[w][0] = pr;
    wsum[w][1] = pk;
    wsum[w][2] = pp;
  }
  __syncthreads();  // also orders the -1 fill before the writes below
  int64_t br = 0, bk = 0, bp = 0;
  for (int x = 0; x < w; ++x) {
    br += wsum[x][0];
    bk += wsum[x][1];
    bp += wsum[x][2];
  }
  int64_t roff = br + pr - rows, koff = bk + pk - kblk, poff = bp + pp - pairs;
  for (int s = s0; s < s1; ++s) {
    int nrb, nkb, np;
    counts(s, nrb, nkb, np);
    a.plan_roff[s] = (int32_t)roff;
    a.plan_roff[ns + s] = (int32_t)koff;
    for (int p = 0; p < np; ++p)
      if (poff + p < a.plan_cap) a.plan_pairs[poff + p] = (s << 7) | p;
    roff += nrb;
    koff += nkb;
    poff += np;
  }
}

// grid (8 * hpx * plan_cap), 512 threads (8 waves, one block-row each).
__global__ __launch_bounds__(512) void k_mapped_av_idx(MappedAvArgs a, int hpx) {
  constexpr int D = 128;
  constexpr int kVBytes = kBlock * D * 2;  // one V block: 16 KB
  __shared__ __attribute__((aligned(16))) uint16_t vst[2][kBlock * D];  // V stages of two columns
  __shared__ int tbl[kIdxRows][kMaxCols];  // stored block of union column x in wave w's row, or -1
  __shared__ int upage[kMaxCols];          // V block (tiled index or page) of union column x
  __shared__ int16_t posu[kMaxCols];       // union index of column c
  __shared__ uint16_t ucol[kMaxCols];      // union columns, ascending
  __shared__ uint8_t anyc[kMaxCols];
  __shared__ int nu_s;
  const int xcd = blockIdx.x % kXcds, m = blockIdx.x / kXcds;
  const int item = m / hpx, hs = xcd * hpx + m % hpx;
  if (hs >= a.n_recv || item >= a.plan_cap) return;
  const int code = ld_const(a.plan_pairs + item);
  if (code < 0) return;
  const int s = code >> 7, pg = code & 127;
  const int32_t n = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
  const int kb0 = chunk_kb0(n, nk);  // block-row r of the queries is block-row kb0 + r of the sequence
  if (!seq_ok(a.vl, s, n, nk) || kb0 < 0) return;
  const int nrb = (n + kBlock - 1) / kBlock, mid = nrb / 2;  // rows mid.. ascending, 0..mid - 1 descending
  const int up_hi = nrb - kIdxRows * pg, up_lo = max(mid, up_hi - kIdxRows);
  if (up_lo >= up_hi) return;
  const int n_pass = kIdxRows * pg < mid ? 2 : 1;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int h = ld_const(a.plan_order + (int64_t)s * a.n_recv + hs);
  const int j = ld_const(a.sender + (int64_t)s * a.sender_stride + h);
  const bool j_ok = j >= 0 && j < a.n_send;
  const int roff = ld_const(a.plan_roff + s), kroff = ld_const(a.plan_roff + a.vl.n_seqs + s);
  const int64_t q0 = cu_q_of(a.vl, s);
  // V of this head's V head: the sequence's tiled key blocks, or the head's page
  // pool (a column's V block is then its page)
  const bool paged = a.v_pages != nullptr;
  const int64_t vg = h / a.v_group;
  const int nkb = (nk + kBlock - 1) / kBlock;
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      a.vt + (paged ? vg * a.v_n_pages : vg * a.n_key_blocks + kroff) * (kBlock * D), (short)0,
      (paged ? a.v_n_pages : nkb) * kVBytes, kBufferFlags);
  const uint32_t a_lane = 32u * (lane & 31) + 16u * (lane >> 5);  // A operand: row L % 32, keys 8 (L / 32) ..
  const uint32_t v_lane = 16u * lane;

  for (int pass = 0; pass < n_pass; ++pass) {
    const bool rev = pass == 1;  // columns descending
    const int lo = rev ? kIdxRows * pg : up_lo, hi = rev ? min(kIdxRows * pg + kIdxRows, mid) : up_hi;
    const int R = lo + wave;  // this wave's block-row (of the queries)
    const bool row_ok = R < hi;
    const int ra_max = kb0 + hi - 1;  // last column of the union
    // this wave's row: stored blocks beg .. end - 1 of its sender
    int beg = 0, end = 0;
    if (j_ok && row_ok) {
      const int64_t gi = (int64_t)j * a.n_block_rows + roff + R;
      beg = ld_const(a.row_ptr + gi);
      end = a.row_end ? ld_const(a.row_end + gi) : ld_const(a.row_ptr + gi + 1);
    }
    // table: union of the rows' kept columns (ascending), and per wave the stored
    // block of each union column
    __syncthreads();  // the previous pass is done with the arrays
    for (int c = tid; c <= ra_max; c += 512) anyc[c] = 0;
    for (int x = lane; x <= ra_max; x += 64) tbl[wave][x] = -1;
    __syncthreads();
    for (int e = beg + lane; e < end; e += 64) {
      const int c = a.col_idx[e];
      if (c >= 0 && c <= kb0 + R) anyc[c] = 1;
    }
    __syncthreads();
    if (wave == 0) {
      int base = 0;
      for (int c0 = 0; c0 <= ra_max; c0 += 64) {
        const int c = c0 + lane;
        const bool f = c <= ra_max && anyc[c];
        const uint64_t mk = __ballot(f);
        if (f) {
          const int x = base + __popcll(mk & ((1ull << lane) - 1ull));
          ucol[x] = (uint16_t)c;
          posu[c] = (int16_t)x;
        }
        base += __popcll(mk);
      }
      if (lane == 0) nu_s = base;
    }
    __syncthreads();
    const int nu = __builtin_amdgcn_readfirstlane(nu_s);
    for (int e = beg + lane; e < end; e += 64) {
      const int c = a.col_idx[e];
      if (c >= 0 && c <= kb0 + R) tbl[wave][posu[c]] = e;
    }
    for (int x = tid; x < nu; x += 512) {
      const int c = ucol[x];
      // a page outside the pool (a broken table) is clamped into it: memory-safe
      upage[x] = paged ? min(max(a.v_pages[(int64_t)s * a.v_page_stride + c], 0), a.v_n_pages - 1)
                       : min(c, nkb - 1);
    }
    __syncthreads();

    f32x16 acc[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[u][dt] = f32x16{};
    if (nu > 0) {
      // union index of sweep step x
      auto xi = [&](int x) __attribute__((always_inline)) { return rev ? nu - 1 - x : x; };
      // stored block of sweep step x in this wave's row (-1: not kept, or x past the end)
      auto blk = [&](int x) __attribute__((always_inline)) { return x < nu ? lds_i32(&tbl[wave][xi(x)]) : -1; };
      // V block of sweep step x into registers: 512 threads x 2 x 16 B; past the
      // end the lane offset lies beyond the descriptor (zeros, no memory access)
      auto load_v = [&](int x, u32x4 (&vr)[2]) __attribute__((always_inline)) {
        const int pgx = x < nu ? lds_i32(&upage[xi(x)]) : 0;
        const uint32_t lo = x < nu ? 16u * tid : kBufferOff;
#pragma unroll
        for (int i = 0; i < 2; ++i) vr[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, lo + 8192u * i, pgx * kVBytes, 0);
      };
      auto store_v = [&](int b, const u32x4 (&vr)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(&vst[b][8 * tid + 4096 * i]) = vr[i];
      };
      // A of panel ks of stored block e (e < 0: a descriptor of no bytes, zeros)
      auto load_a = [&](int e, int ks, u32x4 (&x)[2]) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(a.vals + (int64_t)max(e, 0) * (kBlock * kBlock)), (short)0,
            e >= 0 ? kBlock * kBlock * 2 : 0, kBufferFlags);
#pragma unroll
        for (int u = 0; u < 2; ++u) x[u] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_lane + 1024u * u, 2048 * ks, 0);
      };
      u32x4 A[4][2];  // panel ks of the current column in set ks (ring of four: three panels ahead)
      u32x4 vr[2];
      // prologue: V of step 0 staged, A of its panels 0..2 in flight
      int e_cur = blk(0);
      load_v(0, vr);
      store_v(0, vr);
      load_a(e_cur, 0, A[0]);
      load_a(e_cur, 1, A[1]);
      load_a(e_cur, 2, A[2]);
      barrier_lds();
      for (int x = 0; x < nu; ++x) {
        const int e_nx = blk(x + 1);
        load_v(x + 1, vr);
        const uint32_t vb = lds_addr(&vst[x & 1][0]) + v_lane;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          // panel 4x + ks + 3: panel 3 of this column, or panels 0..2 of the next
          if (ks == 0) load_a(e_cur, 3, A[3]);
          else load_a(e_nx, ks - 1, A[ks - 1]);
          if (e_cur >= 0) {
            u32x4 vo[4];
            asm volatile(
                "ds_read_b128 %0, %4\n"
                "ds_read_b128 %1, %4 offset:1024\n"
                "ds_read_b128 %2, %4 offset:2048\n"
                "ds_read_b128 %3, %4 offset:3072\n"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(vo[0]), "=&v"(vo[1]), "=&v"(vo[2]), "=&v"(vo[3])
                : "v"(vb + 4096u * ks)
                : "memory");
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int dt = 0; dt < 4; ++dt) acc[u][dt] = mfma32(as_bf16x8(A[ks][u]), as_bf16x8(vo[dt]), acc[u][dt]);
          }
        }
        store_v((x + 1) & 1, vr);
        barrier_lds();
        e_cur = e_nx;
      }
    }
    // D[m = row][n = feature]: row = 32 u + 8 (v / 4) + 4 (L / 32) + v % 4, feature = 32 dt + L % 32
    if (row_ok) {
      const int row0 = kBlock * R;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = row0 + 32 * u + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (row >= n) continue;
            const int64_t o = ((int64_t)h * a.vl.total_q + q0 + row) * D + 32 * dt + (lane & 31);
            if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o] = f2bf(acc[u][dt][v]);
            else reinterpret_cast<float*>(a.out)[o] = acc[u][dt][v];
          }
    }
    // drain the stores before the next pass's loads: with stores still counted,
    // the compiler could not size the loop's waits and would drain every step
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
}

// ---------------------------------------------------------------- dense source
// grid (max_q, n_seqs, n_recv); dynamic LDS holds the mixed row, `win` keys at a
// time (the longest key sequence, at most kDenseWin).
constexpr int kDenseWin = 8192;

// 8 consecutive V values starting at element index i as floats; entries at or
// beyond `lim` read 0 (and are not touched in memory).
template <typename T>
__device__ __forceinline__ void ld8(const void* p, int64_t i, int64_t lim, float v[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint16_t* b = reinterpret_cast<const uint16_t*>(p) + i;
    if (lim >= 8 && ((reinterpret_cast<uintptr_t>(b) & 15) == 0)) {
      const u32x4 w = ldg16(b);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(w[e] << 16);
        v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = e < lim ? bf2f(b[e]) : 0.0f;
    }
  } else {
    const float* f = reinterpret_cast<const float*>(p) + i;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < lim ? f[e] : 0.0f;
  }
}

// NT threads, token-major V: 512 (32 key rows per pass, 8 passes unrolled: a row
// streams V with 128 KB of loads outstanding, and two workgroups share a CU) or,
// for launches of few rows, 1024 (64 key rows per pass); key-major V: 256.
template <int D, bool KEY_MAJOR, typename VT, int NT>
// With n_split > 1 (launches of few rows), workgroup x of a row takes the
// split x % n_split of its keys (64-key aligned pieces) and writes its partial
// row to part[split][out element] (fp32); k_dense_split_sum adds the splits.
__global__ __launch_bounds__(NT) void k_mapped_av_dense(MappedAvArgs a, int win, int n_split, float* part) {
  extern __shared__ float bj[];  // mixed row window [win]
  __shared__ int nzi[64];
  __shared__ float nzw[64];
  __shared__ int nnzm;
  __shared__ float red[KEY_MAJOR ? 1 : NT / (D / 8)][D];  // one row per key slot (token-major)
  const int i = blockIdx.x / n_split, sp = blockIdx.x % n_split, s = blockIdx.y, h = blockIdx.z;
  const int32_t nq = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
  if (!seq_ok(a.vl, s, nq, nk) || i >= nq) return;
  const int tid = threadIdx.x;
  const float* Ms = a.M + (int64_t)s * a.M_stride + (int64_t)h * a.n_send;
  // the nonzero mixing weights of this head in ascending sender order (n_send <= 64:
  // one wave loads them together and compacts them with a ballot)
  if (tid < 64) {
    const float w = tid < a.n_send ? Ms[tid] : 0.0f;
    const uint64_t nz = __ballot(w != 0.0f);
    if (w != 0.0f) {
      const int k = __popcll(nz & ((1ull << tid) - 1ull));
      nzi[k] = tid;
      nzw[k] = w;
    }
    if (tid == 0) nnzm = __popcll(nz);
  }
  __syncthreads();
  const int last = nk - nq + i;
  // this workgroup's keys: the whole row, or its split
  int kbeg = 0, kend = last + 1;
  if (n_split > 1) {
    const int chunk = ((last + n_split) / n_split + 63) & ~63;
    kbeg = min(last + 1, sp * chunk);
    kend = min(last + 1, kbeg + chunk);
  }
  const int64_t row_off = map_seq_off(a.vl, s, a.packed) + map_row_off(i, nq, nk, a.packed);
  const int64_t k0 = cu_k_of(a.vl, s);
  // bf16 token-major V whose rows start on 16-byte boundaries takes the
  // pipelined loop in the 1024-thread form (batches of kPipe loads per thread;
  // two batches' registers fit the 128 that 1024 threads allow)
  constexpr int kPipe = (!KEY_MAJOR && NT == 1024 && std::is_same<VT, uint16_t>::value) ? 6 : 0;
  const bool v_al16 = (reinterpret_cast<uintptr_t>(a.v) & 15) == 0;
  constexpr int kChunks = D / 8;          // 8-feature chunks per key (token-major)
  constexpr int kSlots = NT / kChunks;    // keys per pass (token-major)
  float accv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float acck[D / 16];
#pragma unroll
  for (int u = 0; u < D / 16; ++u) acck[u] = 0.0f;
  for (int w0 = kbeg; w0 < kend; w0 += win) {
    const int wlen = min(win, kend - w0);
    for (int j0 = tid; j0 < wlen; j0 += 4 * NT) {
      // four window positions per thread at a time (independent loads)
      float b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int u = 0; u < nnzm; ++u) {
        const int64_t base = (int64_t)nzi[u] * a.head_stride + row_off + w0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int j = j0 + NT * t;
          if (j < wlen)
            b[t] = fmaf(nzw[u], a.maps_bf16 ? bf2f(reinterpret_cast<const uint16_t*>(a.maps)[base + j])
                                            : reinterpret_cast<const float*>(a.maps)[base + j], b[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (j0 + NT * t < wlen) bj[j0 + NT * t] = b[t];
    }
    __syncthreads();
    if constexpr (KEY_MAJOR) {
      // 16 features at a time, 16 threads per feature, 8 keys per 16-byte load
      const int lf = tid & 15, fs = tid >> 4;
#pragma unroll
      for (int rnd = 0; rnd < D / 16; ++rnd) {
        const int f = 16 * rnd + fs;
        const int64_t vrow = ((int64_t)(h / a.v_group) * D + f) * a.vl.total_k + k0 + w0;
        float part = 0.0f;
        for (int j = 8 * lf; j < wlen; j += 128) {
          float v[8];
          ld8<VT>(a.v, vrow + j, wlen - j, v);
#pragma unroll
          for (int e = 0; e < 8; ++e) part = fmaf(j + e < wlen ? bj[j + e] : 0.0f, v[e], part);
        }
        acck[rnd] += part;
      }
    } else if (kPipe > 0 && v_al16) {
      // bf16 V with 1024 threads (a launch of few rows), software-pipelined: a
      // thread's keys are ks, ks + kSlots, ...; they go in batches of kPipe
      // 16-byte loads (kept raw), and the next batch is in flight while the
      // current one is multiplied. Loads past the thread's keys
      // take a lane offset past the descriptor (zeros, no memory access) and
      // weight 0, so the sums equal the unpipelined loop's term for term.
      const int fc = tid % kChunks, ks = tid / kChunks;
      // the window's V rows (uniform: the descriptor lives in scalar registers)
      const uint64_t vaddr = reinterpret_cast<uint64_t>(reinterpret_cast<const uint16_t*>(a.v) +
                                                        ((int64_t)(h / a.v_group) * a.vl.total_k + k0 + w0) * D);
      uint16_t* vwin = reinterpret_cast<uint16_t*>(
          ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(vaddr >> 32)) << 32) |
          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)vaddr));
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          vwin, (short)0, __builtin_amdgcn_readfirstlane(wlen * D * 2), kBufferFlags);
      const int nt = wlen > ks ? (wlen - ks + kSlots - 1) / kSlots : 0;  // this thread's keys
      const int nb = (nt + kPipe - 1) / kPipe;
      // the lane's byte offset in the window; key t of the thread adds the uniform
      // t * kSlots rows as the scalar offset (the range check covers the lane offset)
      const uint32_t vlane = (uint32_t)((ks * D + 8 * fc) * 2);
      u32x4 x0[kPipe > 0 ? kPipe : 1], x1[kPipe > 0 ? kPipe : 1];
      auto load = [&](int b, auto& x) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kPipe; ++u) {
          const int t = kPipe * b + u;
          x[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, t < nt ? vlane : kBufferOff, t * (kSlots * D * 2), 0);
        }
      };
      auto use = [&](int b, const auto& x) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kPipe; ++u) {
          const int t = kPipe * b + u;
          const float bw = t < nt ? bj[min(ks + t * kSlots, wlen - 1)] : 0.0f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            accv[2 * e] = fmaf(bw, __uint_as_float(x[u][e] << 16), accv[2 * e]);
            accv[2 * e + 1] = fmaf(bw, __uint_as_float(x[u][e] & 0xffff0000u), accv[2 * e + 1]);
          }
        }
      };
      if (nb > 0) load(0, x0);
      for (int b = 0; b < nb; b += 2) {
        load(b + 1, x1);  // past the thread's keys: zeros, no memory access
        use(b, x0);
        if (b + 1 < nb) {
          load(b + 2, x0);
          use(b + 1, x1);
        }
      }
    } else {
      // 8 independent 16-byte loads in flight per thread, then their products
      const int fc = tid % kChunks, ks = tid / kChunks;
      const int64_t vbase = ((int64_t)(h / a.v_group) * a.vl.total_k + k0 + w0) * D + 8 * fc;
      int j = ks;
      for (; j + 7 * kSlots < wlen; j += 8 * kSlots) {
        float v[8][8];
#pragma unroll
        for (int u = 0; u < 8; ++u) ld8<VT>(a.v, vbase + (int64_t)(j + u * kSlots) * D, 8, v[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float b = bj[j + u * kSlots];
#pragma unroll
          for (int e = 0; e < 8; ++e) accv[e] = fmaf(b, v[u][e], accv[e]);
        }
      }
      for (; j < wlen; j += kSlots) {
        float v[8];
        ld8<VT>(a.v, vbase + (int64_t)j * D, 8, v);
        const float b = bj[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) accv[e] = fmaf(b, v[e], accv[e]);
      }
    }
    __syncthreads();
  }
  if constexpr (KEY_MAJOR) {
    const int lf = tid & 15, fs = tid >> 4;
#pragma unroll
    for (int rnd = 0; rnd < D / 16; ++rnd) {
      float x = acck[rnd];
      for (int off = 8; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
      if (lf == 0) red[0][16 * rnd + fs] = x;
    }
  } else {
    const int fc = tid % kChunks, ks = tid / kChunks;
#pragma unroll
    for (int e = 0; e < 8; ++e) red[ks][8 * fc + e] = accv[e];
  }
  __syncthreads();
  if (tid < D) {
    float o = 0.0f;
    if constexpr (KEY_MAJOR) {
      o = red[0][tid];
    } else {
      for (int u = 0; u < kSlots; ++u) o += red[u][tid];
    }
    const int64_t oi = ((int64_t)h * a.vl.total_q + cu_q_of(a.vl, s) + i) * D + tid;
    if (n_split > 1) part[(int64_t)sp * a.n_recv * a.vl.total_q * D + oi] = o;
    else if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[oi] = f2bf(o);
    else reinterpret_cast<float*>(a.out)[oi] = o;
  }
}

// The splits of each row added in split order (deterministic). grid (max_q,
// n_seqs, n_recv), D threads.
template <int D>
__global__ __launch_bounds__(D) void k_dense_split_sum(MappedAvArgs a, int n_split, const float* __restrict__ part) {
  const int i = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const int32_t nq = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
  if (!seq_ok(a.vl, s, nq, nk) || i >= nq) return;
  const int64_t oi = ((int64_t)h * a.vl.total_q + cu_q_of(a.vl, s) + i) * D + threadIdx.x;
  const int64_t stride = (int64_t)a.n_recv * a.vl.total_q * D;
  float o = 0.0f;
  for (int sp = 0; sp < n_split; ++sp) o += part[sp * stride + oi];
  if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[oi] = f2bf(o);
  else reinterpret_cast<float*>(a.out)[oi] = o;
}

__global__ void k_onehot(const int32_t* argmax, int64_t rows, int32_t n_send, float* M) {
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= rows * n_send) return;
  const int64_t row = x / n_send;
  const int j = (int)(x % n_send);
  M[x] = argmax[row] == j ? 1.0f : 0.0f;
}

template <int D, bool KM>
static hipError_t dense_launch(const MappedAvArgs& a, hipStream_t st) {
  // the mixed-row window: the longest key sequence (in 64s), at most kDenseWin keys,
  // so that short contexts leave LDS for more workgroups per CU
  const int win = (int)std::min<int64_t>(kDenseWin, std::max<int64_t>(64, ((int64_t)a.max_k + 63) / 64 * 64));
  const size_t lds = (size_t)win * sizeof(float);
  const int64_t rows = (int64_t)a.max_q * a.vl.n_seqs * a.n_recv;
  const int cus = cu_count();
  // A launch of fewer rows than twice the CUs (a long-context decode of a small
  // batch) splits each row's keys over up to kDenseSplitMax workgroups (at least
  // 1024 keys each, at most two workgroups per CU in all) when the workspace
  // holds the partial rows.
  int n_split = 1;
  if (rows < 2 * (int64_t)cus && a.part) {
    n_split = (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)kDenseSplitMax, 2 * (int64_t)cus / rows,
                                                           (int64_t)a.max_k / 1024}));
    if ((size_t)n_split * a.n_recv * a.vl.total_q * D * sizeof(float) > a.part_bytes) n_split = 1;
  }
  dim3 grid((unsigned)(a.max_q * n_split), (unsigned)a.vl.n_seqs, (unsigned)a.n_recv);
  {
    KernelTimer kt_("k_mapped_av_dense", st);
    // token-major V, unsplit: with few rows 1024 threads keep more loads in
    // flight per row; otherwise 512 threads let two workgroups share a CU
    bool big = false;
    if constexpr (!KM) big = n_split == 1 && rows < 2 * (int64_t)cus;
    if (big) {
      if (a.v_bf16) hipLaunchKernelGGL((k_mapped_av_dense<D, KM, uint16_t, 1024>), grid, dim3(1024), lds, st, a, win, n_split, a.part);
      else hipLaunchKernelGGL((k_mapped_av_dense<D, KM, float, 1024>), grid, dim3(1024), lds, st, a, win, n_split, a.part);
    } else {
      constexpr int NT = KM ? 256 : 512;
      if (a.v_bf16) hipLaunchKernelGGL((k_mapped_av_dense<D, KM, uint16_t, NT>), grid, dim3(NT), lds, st, a, win, n_split, a.part);
      else hipLaunchKernelGGL((k_mapped_av_dense<D, KM, float, NT>), grid, dim3(NT), lds, st, a, win, n_split, a.part);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_split == 1) return e;
  {
    KernelTimer kt_("k_dense_split_sum", st);
    hipLaunchKernelGGL((k_dense_split_sum<D>), dim3((unsigned)a.max_q, (unsigned)a.vl.n_seqs, (unsigned)a.n_recv),
                       dim3(D), 0, st, a, n_split, a.part);
  }
  return hipGetLastError();
}

hipError_t launch_mapped_av_dense(const MappedAvArgs& a, hipStream_t st) {
  if (a.n_recv == 0 || a.vl.n_seqs == 0 || a.max_q == 0) return hipSuccess;
  if (a.v_key_major) return a.d == 64 ? dense_launch<64, true>(a, st) : dense_launch<128, true>(a, st);
  return a.d == 64 ? dense_launch<64, false>(a, st) : dense_launch<128, false>(a, st);
}

hipError_t launch_tile_v(const MappedAvArgs& a, hipStream_t st) {
  if (a.n_v == 0 || a.vl.n_seqs == 0 || a.max_k == 0) return hipSuccess;
  const int nkb = (a.max_k + 63) / 64;
  dim3 tg((unsigned)nkb, a.vl.n_seqs, a.n_v);  // each V head once
  KernelTimer kt_("k_tile_v", st);
  if (a.v_key_major)
    hipLaunchKernelGGL(k_tile_v<true>, tg, dim3(256), 0, st, reinterpret_cast<const uint16_t*>(a.v), a.vt, a.vl,
                       a.n_key_blocks, a.v_pages, a.v_page_stride, a.v_n_pages);
  else
    hipLaunchKernelGGL(k_tile_v<false>, tg, dim3(256), 0, st, reinterpret_cast<const uint16_t*>(a.v), a.vt, a.vl,
                       a.n_key_blocks, a.v_pages, a.v_page_stride, a.v_n_pages);
  return hipGetLastError();
}

hipError_t launch_mapped_av_bsr(const MappedAvArgs& a, hipStream_t st) {
  if (a.n_recv == 0 || a.vl.n_seqs == 0 || a.max_q == 0) return hipSuccess;
  const int nrb = (a.max_q + 63) / 64;
  if (!a.v_tiled) {
    hipError_t e = launch_tile_v(a, st);
    if (e != hipSuccess) return e;
  }
  const int n_hg = (a.n_recv + kHeadsPerWg - 1) / kHeadsPerWg;
  const int hpg = (a.n_recv + n_hg - 1) / n_hg;
  const int n_pairs = (nrb + 1) / 2;  // block-rows R - 1 - p and p
  const int64_t units = (int64_t)n_pairs * a.vl.n_seqs;
  const int64_t rounds = (units + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(rounds * kXcds * 2 * n_hg));
  // More senders than one workgroup stages: one pass per group of kSend senders,
  // each later pass adding its product to the output (the mix is linear in M).
  for (int j0 = 0; j0 < a.n_send; j0 += kSend) {
    MappedAvArgs g = a;
    g.send0 = j0;
    g.n_send = min(kSend, a.n_send - j0);
    g.m_ld = a.n_send;
    g.accum = j0 > 0;
    {
      KernelTimer kt_("k_mapped_av_bsr", st);
      hipLaunchKernelGGL(k_mapped_av_bsr, grid, dim3(kThreads), 0, st, g, n_pairs, n_hg, hpg);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_mapped_av_indexed(const MappedAvArgs& a, hipStream_t st) {
  if (a.n_recv == 0 || a.vl.n_seqs == 0 || a.max_q == 0) return hipSuccess;
  if (!a.v_tiled) {
    hipError_t e = launch_tile_v(a, st);
    if (e != hipSuccess) return e;
  }
  {
    KernelTimer kt_("k_idx_order", st);
    hipLaunchKernelGGL(k_idx_order, dim3((unsigned)a.vl.n_seqs), dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    KernelTimer kt_("k_idx_plan", st);
    hipLaunchKernelGGL(k_idx_plan, dim3(1), dim3(kPlanThreads), 0, st, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int hpx = (a.n_recv + kXcds - 1) / kXcds;  // heads per XCD
  {
    KernelTimer kt_("k_mapped_av_idx", st);
    hipLaunchKernelGGL(k_mapped_av_idx, dim3((unsigned)(kXcds * hpx * a.plan_cap)), dim3(512), 0, st, a, hpx);
  }
  return hipGetLastError();
}

hipError_t launch_onehot(const int32_t* argmax, int32_t n_batch, int32_t n_recv, int32_t n_send,
                         float* M, hipStream_t st) {
  const int64_t tot = (int64_t)n_batch * n_recv * n_send;
  if (tot == 0) return hipSuccess;
  KernelTimer kt_("k_onehot", st);
  hipLaunchKernelGGL(k_onehot, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, argmax,
                     (int64_t)n_batch * n_recv, n_send, M);
  return hipGetLastError();
}

}  // namespace cma
