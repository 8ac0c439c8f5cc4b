// Two-phase block-sparse compression of causal maps (MapFlow, storage and
// execution): phase 1 gathers 64x64 block statistics in one QK^T sweep per
// block-row and selects the blocks to keep; phase 2 recomputes only the kept
// blocks and writes them. The dense map is never formed.
//
// Both phases give a workgroup a group of G adjacent block-rows (G = 2, so 128
// queries share every staged K block; phase 1 falls back to G = 1 when its
// per-(query, block) table for two rows would not fit in LDS, above 128
// block-rows). Its 8 waves are 2G query tiles of 32 queries x 8 / (2G) key
// phases; each K round stages 4 key blocks and a wave takes 2G / 2 of them.
//
// Phase 1 (k_block_stats): for every (query, key block) the online softmax
// leaves a partial sum relative to the running max at that block; log2 of the
// absolute partial goes to LDS. After the sweep the running statistics of the
// key phases are merged into each query's final (max, sum), and the mass of
// block c is
//   mass_c = sum_i partial_ic * 2^(max_ic - max_i) / sum_i
// added over the 64 query rows of its block-row in a fixed order (four partial
// sums of 16 rows, then combined pairwise). Selection (normalise by the
// block-row total, order largest first with ties to the lower column, keep the
// shortest prefix whose running sum reaches tau) runs in the same workgroup:
// every block's rank comes from wave-wide ballots over all weights, and one
// wave scans the running sum.
// Scan (k_bsr_scan): exclusive scan of kept counts -> row_ptr, nnz.
// Phase 2 (k_block_extract): the union of the group's kept columns is swept;
// a wave recomputes the blocks its block-row kept, p = 2^(t - lse2), and
// stores them as bf16 with their column indices.
#include <type_traits>

#include "kernels.hpp"
#include "score.hpp"

namespace cma {

// Work item of workgroup `id`: (head h, sequence s, row group rg = block-rows
// G rg .. G rg + G - 1). The hardware deals workgroup ids round-robin over the
// 8 XCDs (id i runs on XCD i % 8, as that XCD's (i / 8)-th workgroup). With
// enough (head, sequence) pairs they are dealt the same way: an XCD walks the
// row groups of one pair at a time, longest first, and its L2 keeps that pair's
// K, which every row group of the pair re-reads. With few pairs (fewer than 2
// per XCD) that would idle XCDs, so ids then go pair by pair. Grid:
// group_grid() workgroups.
__device__ __forceinline__ bool group_item(int id, int ngr, int n_seqs, int n_heads, int& h, int& s, int& rg) {
  const int pairs = n_seqs * n_heads;
  int pair, j;
  if (pairs >= 2 * kXcds) {
    const int xcd = id % kXcds;
    j = id / kXcds;
    pair = xcd + kXcds * (j / ngr);
  } else {
    j = id;
    pair = id / ngr;
  }
  if (pair >= pairs) return false;
  h = pair / n_seqs;
  s = pair % n_seqs;
  rg = ngr - 1 - j % ngr;
  return true;
}

inline unsigned group_grid(int ngr, int n_seqs, int n_heads) {
  const int64_t pairs = (int64_t)n_seqs * n_heads;
  if (pairs < 2 * kXcds) return (unsigned)(pairs * ngr);
  return (unsigned)(kXcds * ((pairs + kXcds - 1) / kXcds) * ngr);
}

// Block statistics and selection for one (head, sequence, row group).
// Dynamic LDS: two K stages, then LP[64 G][LPS] = log2 of each (query, block)
// partial sum in absolute terms (running max + log2 of the partial), so that
// mass_c = sum_i 2^(LP[i][c] - lse_i) once the row's lse is known.
template <int D, int G>
__global__ __launch_bounds__(512) void k_block_stats(CompressArgs a) {
  constexpr int QT = 2 * G, KP = 8 / QT, BPW = 4 / KP;  // query tiles, key phases, blocks per wave and round
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  // row stride of LP: odd, so the 32 query rows written for one block fall in
  // distinct LDS banks
  const int LPS = (a.ncb_max + 1) | 1;
  uint8_t* stage = reinterpret_cast<uint8_t*>(dyn);
  float* LP = dyn + 2 * (kStageBytes / 4);
  __shared__ float sm[KP][64 * G], sl[KP][64 * G];
  __shared__ float lse_s[64 * G];
  __shared__ float mass_a[G][kMaxBlockRows];
  __shared__ float wts_a[G][kMaxBlockRows];  // weights in column order, then in rank order
  __shared__ int order_a[G][kMaxBlockRows];
  __shared__ __attribute__((aligned(16))) uint64_t key_a[G][kMaxBlockRows];
  __shared__ uint32_t kept_a[G][kWords];
  __shared__ int kcount_a[G];
  __shared__ float total_a[G];

  int h, s, rg;
  if (!group_item(blockIdx.x, (a.nrb_max + G - 1) / G, a.vl.n_seqs, a.n_heads, h, s, rg)) return;
  // n query rows at the end of nk keys (a chunk; n = nk for a whole prompt):
  // block-row r of the chunk is block-row kb0 + r of the sequence's grid
  const int32_t n = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
  const int kb0 = chunk_kb0(n, nk);
  const int nrb = (n + kBlock - 1) / kBlock, r0 = G * rg;
  if (!seq_ok(a.vl, s, n, nk) || kb0 < 0 || r0 >= nrb) return;
  const int r_last = min(r0 + G - 1, nrb - 1);
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int qt = wave % QT, kp = wave / QT;
  const int rq = kb0 + r0 + qt / 2;                       // the tile's block-row in the sequence's grid
  const int c_last = kb0 + r_last;                        // last key block of the group
  const int cmax = rq <= c_last ? rq : -1;                // last key block the tile computes
  const int qloc = 64 * (qt / 2) + 32 * (qt & 1) + (lane & 31);  // query within the group
  const int i = 64 * r0 + qloc;                           // query row within the chunk
  const bool valid = i < n;
  const int ipos = 64 * kb0 + i;                          // its key position
  const uint16_t* qrow = a.q + ((int64_t)h * a.vl.total_q + cu_q_of(a.vl, s) + min(i, n - 1)) * D;
  const uint16_t* kseq = a.k + ((int64_t)h * a.vl.total_k + cu_k_of(a.vl, s)) * D;
  const float scale_l2 = ld_const(a.scale + h) * kLog2e;
  const float bias_l2 = a.bias ? ld_const(a.bias + h) * kLog2e : 0.0f;

  QOperand<D> qop;
  load_query_clamped<D>(qop, qrow, valid);
  f32x16 acc[BPW][2];
  float m = -INFINITY, l = 0.0f;
  // Blocks strictly between column 0 (sink bias) and the diagonal (causal mask)
  // take the lean update on raw scores.
  const bool raw_ok = scale_l2 > 0.0f;
  auto finish = [&](f32x16 (&x)[2], int c) __attribute__((always_inline)) {
    float part;
    if (raw_ok && c != 0 && c != rq) {
      part = online_update_raw(x, scale_l2, m, l);
    } else {
      logits_inplace(x, 64 * c, valid ? ipos : -1, scale_l2, bias_l2);
      part = online_update_acc(x, m, l);
    }
    if (lane < 32) LP[qloc * LPS + c] = m + log2f_fast(part);
  };
  // Round k stages blocks 4k .. 4k + 3; the wave takes blocks 4k + kp + KP j.
  if constexpr (BPW == 1) {
    kstage_pipeline<D>(
        stage, kseq, nk, (c_last + 4) / 4, [&](int c) { return 64 * min(c, c_last); },
        [&](int k, const uint8_t* buf, auto fh) {
          constexpr int FH = decltype(fh)::value;
          const int c = 4 * k + kp;
          if (c > cmax) return;
          if (FH == 0) acc[0][0] = acc[0][1] = f32x16{};
          kstage_mma<D, FH>(acc[0], buf + kp * kStageBlockBytes, qop);
          if (FH == D / 64 - 1) finish(acc[0], c);
        });
  } else {
    // Two whole blocks per sub-step (kstage2_pipeline): the wave computes block
    // 2u + kp of sub-step u and runs its softmax update in sub-step u + 1, beside
    // that sub-step's products, so every sub-step has matrix and vector work.
    // The two accumulator sets alternate with the sub-step's parity.
    constexpr int FHN = D / 64;
    int c_def = -1;  // block computed in the previous sub-step, or -1
    auto sub = [&](int u, const uint8_t* buf, auto par) __attribute__((always_inline)) {
      constexpr int P = decltype(par)::value;
      const int c = 2 * u + kp;
      if (c <= cmax && c_def >= 0 && raw_ok && c_def != 0 && c_def != rq) {
        // interior: this block's products beside the previous block's lean update
        const float part = mma_beside_update<D>(acc[P], buf + kp * FHN * kStageBlockBytes, qop, acc[1 - P], scale_l2, m, l);
        if (lane < 32) LP[qloc * LPS + c_def] = m + log2f_fast(part);
      } else {
        if (c <= cmax) {
          acc[P][0] = acc[P][1] = f32x16{};
          kstage_mma<D, 0>(acc[P], buf + kp * FHN * kStageBlockBytes, qop);
          if constexpr (FHN == 2) kstage_mma<D, 1>(acc[P], buf + (2 * kp + 1) * kStageBlockBytes, qop);
        }
        if (c_def >= 0) finish(acc[1 - P], c_def);
      }
      c_def = c <= cmax ? c : -1;
    };
    const int nsub = (c_last + 2) / 2;
    kstage2_pipeline<D>(stage, kseq, nk, nsub, [&](int c) { return 64 * min(c, c_last); },
                        [&](int u, const uint8_t* buf) {
                          if (u & 1) sub(u, buf, std::integral_constant<int, 1>{});
                          else sub(u, buf, std::integral_constant<int, 0>{});
                        });
    if (c_def >= 0) {
      if ((nsub - 1) & 1) finish(acc[1], c_def);
      else finish(acc[0], c_def);
    }
  }
  if (lane < 32) {
    sm[kp][qloc] = m;
    sl[kp][qloc] = l;
  }
  __syncthreads();
  if (tid < 64 * G) {
    const int q = tid;
    float M = -INFINITY;
    for (int w = 0; w < KP; ++w) M = fmaxf(M, sm[w][q]);
    float L = 0.0f;
    for (int w = 0; w < KP; ++w)
      if (sm[w][q] != -INFINITY) L += sl[w][q] * exp2f_fast(sm[w][q] - M);
    const float lse = M + log2f_fast(L);
    lse_s[q] = lse;
    const int iq = 64 * r0 + q;
    if (iq < n) {
      const int64_t tok = (int64_t)h * a.vl.total_q + cu_q_of(a.vl, s) + iq;
      a.lse2[tok] = lse;
      if (a.row_stats) {
        a.row_stats[2 * tok] = M * kLn2;
        a.row_stats[2 * tok + 1] = L;
      }
    }
  }

  // Selection, the group's rows side by side: waves 4 gr .. 4 gr + 3 (all 8
  // waves when G = 1) take block-row r0 + gr.
  constexpr int NTR = 512 / G, NWR = NTR / 64;  // threads and waves per row
  const int gr = wave / NWR, tl = tid % NTR, wl = wave % NWR;
  const int r = r0 + gr;
  const bool act = r <= r_last;
  float* mass = mass_a[gr];
  float* wts = wts_a[gr];
  int* order = order_a[gr];
  uint64_t* key = key_a[gr];
  uint32_t* kept = kept_a[gr];
  int32_t roff, kroff;
  int64_t tri_off;
  bsr_offsets(a.vl, s, roff, kroff, tri_off);
  __syncthreads();  // lse_s is written
  if (tl < kWords) kept[tl] = 0u;
  // mass_c over the valid rows: four consecutive threads take rows 16 part ..
  // + 15 of block c, then add their partials in a fixed order
  const int nrows = act ? min(64, n - 64 * r) : 0;
  const int nb = act ? kb0 + r + 1 : 0;
  const float* LPr = LP + 64 * gr * LPS;
  const float* lser = lse_s + 64 * gr;
  // (every thread reads its 16 entries, those of a column past the row's last
  // read a valid one, so that the reads are all in flight at once; rows past the
  // sequence end then add nothing)
  for (int x0 = 0; x0 < 4 * nb; x0 += NTR) {
    const int x = x0 + tl, c = x >> 2, part = x & 3;
    const int cc = min(c, nb - 1);
    float t[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) t[e] = LPr[(16 * part + e) * LPS + cc] - lser[16 * part + e];
    float y = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) y += 16 * part + e < nrows ? exp2f_fast(t[e]) : 0.0f;
    y += __shfl_xor(y, 1, 64);  // (p0 + p1), (p2 + p3)
    y += __shfl_xor(y, 2, 64);  // (p0 + p1) + (p2 + p3)
    if (c < nb && part == 0) mass[c] = y;
  }
  __syncthreads();

  const int64_t g = (int64_t)h * a.n_block_rows + roff + r;
  if (act && a.block_mass) {
    int32_t r_all, kr_all;
    int64_t n_tri;  // blocks per head over all sequences
    bsr_offsets(a.vl, a.vl.n_seqs, r_all, kr_all, n_tri);
    float* bm = a.block_mass + (int64_t)h * n_tri + tri_off + (int64_t)r * kb0 + (int64_t)r * (r + 1) / 2;
    for (int c = tl; c < nb; c += NTR) bm[c] = mass[c];
  }
  if (a.tau >= 1.0f) {
    for (int c = tl; c < nb; c += NTR) atomicOr(&kept[c >> 5], 1u << (c & 31));
    if (tl == 0) kcount_a[gr] = nb;
  } else {
    // total mass: one wave per row, strided partial sums then a fixed lane tree
    if (wl == 0) {
      float x = 0.0f;
      for (int c = lane; c < nb; c += 64) x += mass[c];
      x = wave_scan_add(x);
      if (lane == 63) total_a[gr] = x;
    }
    __syncthreads();
    const float total = total_a[gr];
    // Weights, and sort keys: a weight's bits (nonnegative floats order as
    // unsigned integers) above the complemented column, so that one unsigned
    // comparison orders blocks weight descending, column ascending. A NaN weight
    // (only from non-finite inputs) ranks as 0, so that the order stays a strict
    // total order and the kept set a set of columns of this row with exactly
    // kcount members. Slots from nb up to the next multiple of 16 get key 0,
    // which no block's key is below.
    const int nb16 = (nb + 15) & ~15;
    for (int c = tl; c < nb16; c += NTR) {
      const float w = c < nb ? mass[c] / total : 0.0f;
      const float wv = w == w ? w : 0.0f;
      key[c] = c < nb ? ((uint64_t)__float_as_uint(wv) << 32) | (uint64_t)(0xffffffffu - (uint32_t)c) : 0ull;
    }
    __syncthreads();
    // rank of block c = the number of blocks ahead of it: each thread of the row
    // takes its blocks and compares their keys with every key of the row (16 per
    // step, all lanes reading the same key: broadcast reads); the block's weight
    // goes to its rank's slot
    for (int c = tl; c < nb; c += NTR) {
      const uint64_t kc = key[c];
      int rank = 0;
      for (int c2 = 0; c2 < nb16; c2 += 16) {
        uint64_t k16[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) k16[e] = key[c2 + e];
#pragma unroll
        for (int e = 0; e < 16; ++e) rank += (int)(k16[e] > kc);
      }
      order[rank] = c;
      wts[rank] = __uint_as_float((uint32_t)(kc >> 32));
    }
    __syncthreads();
    // running sum in that order (one wave per row: 4 consecutive ranks per lane,
    // then a wave-wide inclusive scan of the lane totals); keep the shortest
    // prefix whose sum reaches tau
    if (wl == 0 && act) {
      float cum[4];
      float run = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int x = 4 * lane + e;
        run += x < nb ? wts[x] : 0.0f;
        cum[e] = run;
      }
      const float before = wave_scan_add(run) - run;
      int mine = 4 * 64;
#pragma unroll
      for (int e = 3; e >= 0; --e)
        if (4 * lane + e < nb && before + cum[e] >= a.tau) mine = 4 * lane + e;
      // the running sum only grows: the first rank that reaches tau is the
      // lowest lane's hit
      const uint64_t hit = __ballot(mine < 4 * 64);
      const int first = hit ? __builtin_amdgcn_readlane(mine, (int)__builtin_ctzll(hit)) : 4 * 64;
      if (lane == 0) kcount_a[gr] = first < nb ? first + 1 : nb;
    }
    __syncthreads();
    for (int x = tl; x < (act ? kcount_a[gr] : 0); x += NTR) {
      const int c = order[x];
      atomicOr(&kept[c >> 5], 1u << (c & 31));
    }
  }
  __syncthreads();
  if (act) {
    if (tl < kWords) a.kept[g * kWords + tl] = kept[tl];
    if (tl == 0) a.counts[g] = kcount_a[gr];
  }
}

// Exclusive scan of the kept counts (one workgroup). The counts go through LDS
// in tiles of kScanTile with coalesced loads and stores; each thread scans 8
// consecutive counts, a wave scan and the 16 wave totals give its offset, and a
// carry runs across tiles. Deterministic (integers).
constexpr int kScanThreads = 1024, kScanPer = 8, kScanTile = kScanThreads * kScanPer;

__global__ __launch_bounds__(kScanThreads) void k_bsr_scan(const int32_t* counts, int64_t n,
                                                           int32_t* row_ptr, int32_t* nnz) {
  __shared__ __attribute__((aligned(16))) int32_t buf[kScanTile];
  __shared__ int64_t wsum[kScanThreads / 64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int64_t carry = 0;
  for (int64_t base = 0; base < n; base += kScanTile) {
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      const int64_t x = base + i * kScanThreads + t;
      buf[i * kScanThreads + t] = x < n ? counts[x] : 0;
    }
    __syncthreads();
    const int4 c0 = reinterpret_cast<const int4*>(buf)[2 * t];
    const int4 c1 = reinterpret_cast<const int4*>(buf)[2 * t + 1];
    const int32_t v[kScanPer] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    int64_t own = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) own += v[i];
    int64_t pre = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(pre, off, 64);
      if (lane >= off) pre += y;
    }
    if (lane == 63) wsum[w] = pre;
    __syncthreads();
    int64_t before = 0, total = 0;
#pragma unroll
    for (int j = 0; j < kScanThreads / 64; ++j) {
      const int64_t sj = wsum[j];
      before += j < w ? sj : 0;
      total += sj;
    }
    int64_t run = carry + before + pre - own;
    int32_t o[kScanPer];
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      o[i] = (int32_t)run;
      run += v[i];
    }
    reinterpret_cast<int4*>(buf)[2 * t] = make_int4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<int4*>(buf)[2 * t + 1] = make_int4(o[4], o[5], o[6], o[7]);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      const int64_t x = base + i * kScanThreads + t;
      if (x < n) row_ptr[x] = buf[i * kScanThreads + t];
    }
    carry += total;
    __syncthreads();  // buf and wsum are rewritten by the next tile
  }
  if (t == 0) {
    row_ptr[n] = (int32_t)carry;
    nnz[0] = (int32_t)carry;
  }
}

// Extraction of the kept blocks of one (head, sequence, row group of 2
// block-rows): the union of the two rows' kept columns is swept 2 columns per
// sub-step; wave (qt, kp) recomputes, for its 32 query rows, column 2u + kp of
// sub-step u if its block-row kept it.
template <int D>
__global__ __launch_bounds__(512) void k_block_extract(CompressArgs a) {
  constexpr int G = 2, QT = 4;
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  uint8_t* stage = reinterpret_cast<uint8_t*>(dyn);
  __shared__ int ucols[kMaxBlockRows];     // kept columns of either row, ascending
  __shared__ int bidx[G][kMaxBlockRows];   // block index of union entry x in row gr, or -1
  __shared__ int nu_s;
  int h, s, rg;
  if (!group_item(blockIdx.x, (a.nrb_max + G - 1) / G, a.vl.n_seqs, a.n_heads, h, s, rg)) return;
  const int32_t n = seq_len_q(a.vl, s), nk = seq_len_k(a.vl, s);
  const int kb0 = chunk_kb0(n, nk);  // the chunk's first block-row in the sequence's grid
  const int nrb = (n + kBlock - 1) / kBlock, r0 = G * rg;
  if (!seq_ok(a.vl, s, n, nk) || kb0 < 0 || r0 >= nrb) return;
  if ((int64_t)a.nnz[0] > a.capacity) return;
  const int r_last = min(r0 + G - 1, nrb - 1);
  int32_t roff, kroff;
  int64_t tri_off;
  bsr_offsets(a.vl, s, roff, kroff, tri_off);
  const int64_t g0 = (int64_t)h * a.n_block_rows + roff + r0;  // row r0; row r0 + 1 is g0 + 1
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  if (wave == 0) {
    // union of the kept masks in ascending column order, each row's rank of a
    // column among its own kept columns, and the rows' column indices
    const bool has1 = r0 + 1 <= r_last;
    const int64_t p0 = a.row_ptr[g0], p1 = has1 ? a.row_ptr[g0 + 1] : 0;
    int nu = 0, k0 = 0, k1 = 0;
    for (int c0 = 0; c0 < kMaxBlockRows; c0 += 64) {
      const int c = c0 + lane, w = c >> 5;
      const bool b0 = (a.kept[g0 * kWords + w] >> (c & 31)) & 1u;
      const bool b1 = has1 && ((a.kept[(g0 + 1) * kWords + w] >> (c & 31)) & 1u);
      const uint64_t below = (1ull << lane) - 1ull;
      const uint64_t mu = __ballot(b0 || b1), m0 = __ballot(b0), m1 = __ballot(b1);
      const int x = nu + __popcll(mu & below), i0 = k0 + __popcll(m0 & below), i1 = k1 + __popcll(m1 & below);
      if (b0 || b1) {
        ucols[x] = c;
        bidx[0][x] = b0 ? i0 : -1;
        bidx[1][x] = b1 ? i1 : -1;
      }
      if (b0) a.col_idx[p0 + i0] = c;
      if (b1) a.col_idx[p1 + i1] = c;
      nu += __popcll(mu);
      k0 += __popcll(m0);
      k1 += __popcll(m1);
    }
    if (lane == 0) nu_s = nu;
  }
  __syncthreads();
  const int nu = nu_s;
  if (nu == 0) return;
  const int qt = wave % QT, kp = wave / QT, gr = qt / 2;
  const int rq = r0 + gr;                      // the tile's block-row (in the chunk)
  const int rq_abs = kb0 + rq;                 // and in the sequence's grid
  const bool tile_ok = rq <= r_last;
  const int iloc = 32 * (qt & 1) + (lane & 31);
  const int i = 64 * rq + iloc;
  const bool valid = tile_ok && i < n;
  const int ipos = 64 * kb0 + i;               // the query's key position
  const int half = lane >> 5;
  const uint16_t* qrow = a.q + ((int64_t)h * a.vl.total_q + cu_q_of(a.vl, s) + min(i, n - 1)) * D;
  const uint16_t* kseq = a.k + ((int64_t)h * a.vl.total_k + cu_k_of(a.vl, s)) * D;
  const float scale_l2 = ld_const(a.scale + h) * kLog2e;
  const float bias_l2 = a.bias ? ld_const(a.bias + h) * kLog2e : 0.0f;
  const float lse = valid ? a.lse2[(int64_t)h * a.vl.total_q + cu_q_of(a.vl, s) + i] : 0.0f;
  const int64_t base = tile_ok ? ld_const(a.row_ptr + g0 + gr) : 0;  // written by the scan before this kernel
  QOperand<D> qop;
  load_query_clamped<D>(qop, qrow, valid);
  f32x16 acc[2][2];
  const bool raw_ok = scale_l2 > 0.0f;
  // block index (in this tile's row) of union entry x, or -1 (not kept, or past the end)
  auto blk_of = [&](int x) __attribute__((always_inline)) {
    return (tile_ok && x < nu) ? __builtin_amdgcn_readfirstlane(bidx[gr][x]) : -1;
  };
  // p = 2^(logit - lse) in the accumulators (0 for rows past the end)
  auto finish = [&](f32x16 (&x)[2], int c) __attribute__((always_inline)) {
    if (raw_ok && c != 0 && c != rq_abs) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) x[kt][v] = exp2f_fast(fmaf(x[kt][v], scale_l2, -lse));
    } else {
      logits_inplace(x, 64 * c, valid ? ipos : -1, scale_l2, bias_l2);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) x[kt][v] = exp2f_fast(x[kt][v] - lse);
    }
    if (!valid) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) x[kt] = f32x16{};
    }
  };
  // x as bf16 into block b of the row; b < 0: the same stores through a
  // descriptor of zero bytes, which write nothing. Every sub-step thus issues the
  // same stores, so the compiler's wait for the next stage's K (loaded before
  // them) does not also wait for them.
  auto store_block = [&](const f32x16 (&x)[2], int b) __attribute__((always_inline)) {
    // Lane (query, half) holds keys 32kt + 8g + 4half + 0..3 for g = 0..3. One
    // exchange with the partner lane (lane ^ 32) per pair of groups leaves lane
    // half h with the 8 consecutive keys 32kt + 16g2 + 8h .. +7, so that each
    // store writes 16 bytes and one instruction fills a whole 1 KB run of a
    // panel (32 rows x 16 keys).
    uint16_t* blk = b >= 0 ? a.vals + (base + b) * (int64_t)(kBlock * kBlock) : a.vals;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(blk, (short)0, b >= 0 ? 2 * kBlock * kBlock : 0, kBufferFlags);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const int v0 = 8 * g2;  // elements v0..v0+3 (group 2g2), v0+4..v0+7 (group 2g2+1)
        const uint32_t x0 = pack2bf(x[kt][v0], x[kt][v0 + 1]);
        const uint32_t x1 = pack2bf(x[kt][v0 + 2], x[kt][v0 + 3]);
        const uint32_t y0 = pack2bf(x[kt][v0 + 4], x[kt][v0 + 5]);
        const uint32_t y1 = pack2bf(x[kt][v0 + 6], x[kt][v0 + 7]);
        // lanes 0-31 keep x and receive the partner's x; lanes 32-63 receive
        // the partner's y and keep their own y
        const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
        const u32x4 w = {s0[0], s1[0], s0[1], s1[1]};
        const int panel = 2 * kt + g2;
        // non-temporal (cache policy nt): the blocks are not read again here, and
        // 7.8 GB of them streaming through L2 would otherwise evict the K that is re-read
        __builtin_amdgcn_raw_buffer_store_b128(w, rs, 2u * (uint32_t)(panel * (kBlock * kPanel) + iloc * kPanel + 8 * half), 0,
                                               kCacheNT);
      }
  };
  // Whole-block sub-steps (kstage2_pipeline): the wave computes union entry
  // 2u + kp of sub-step u if its block-row kept it, and exponentiates and stores
  // it in sub-step u + 1, beside that sub-step's products. The two accumulator
  // sets alternate with the sub-step's parity.
  constexpr int FHN = D / 64;
  int x_def = -1, b_def = -1;  // entry computed in the previous sub-step and its block index
  auto sub = [&](int u, const uint8_t* buf, auto par) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    const int x = 2 * u + kp, b = blk_of(x);
    if (b >= 0) {
      acc[P][0] = acc[P][1] = f32x16{};
      kstage_mma<D, 0>(acc[P], buf + kp * FHN * kStageBlockBytes, qop);
      if constexpr (FHN == 2) kstage_mma<D, 1>(acc[P], buf + (2 * kp + 1) * kStageBlockBytes, qop);
    }
    if (b_def >= 0) finish(acc[1 - P], ucols[x_def]);
    store_block(acc[1 - P], b_def);
    x_def = x;
    b_def = b;
  };
  const int nsub = (nu + 1) / 2;
  kstage2_pipeline<D>(
      stage, kseq, nk, nsub, [&](int x) { return 64 * ucols[min(x, nu - 1)]; },
      [&](int u, const uint8_t* buf) {
        if (u & 1) sub(u, buf, std::integral_constant<int, 1>{});
        else sub(u, buf, std::integral_constant<int, 0>{});
      },
      [&] { store_block(acc[0], -1); });
  if (b_def >= 0) {
    if ((nsub - 1) & 1) {
      finish(acc[1], ucols[x_def]);
      store_block(acc[1], b_def);
    } else {
      finish(acc[0], ucols[x_def]);
      store_block(acc[0], b_def);
    }
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
  // phase 1 takes two block-rows per workgroup when their per-(query, block)
  // table fits in LDS next to the K stages, else one
  const bool two = a.ncb_max <= 128;
  const int G = two ? 2 : 1;
  const int lps = (a.ncb_max + 1) | 1;
  const size_t lds = 2 * (size_t)kStageBytes + (size_t)64 * G * lps * sizeof(float);
  const dim3 grid(group_grid((a.nrb_max + G - 1) / G, a.vl.n_seqs, a.n_heads));
  const void* fn = two ? reinterpret_cast<const void*>(&k_block_stats<D, 2>)
                       : reinterpret_cast<const void*>(&k_block_stats<D, 1>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  {
    KernelTimer kt_("k_block_stats", st);
    if (two) hipLaunchKernelGGL((k_block_stats<D, 2>), grid, dim3(512), lds, st, a);
    else hipLaunchKernelGGL((k_block_stats<D, 1>), grid, dim3(512), lds, st, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    KernelTimer kt_("k_bsr_scan", st);
    hipLaunchKernelGGL(k_bsr_scan, dim3(1), dim3(kScanThreads), 0, st, a.counts,
                       (int64_t)a.n_heads * a.n_block_rows, a.row_ptr, a.nnz);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds_x = 2 * (size_t)kStageBytes;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_block_extract<D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_x);
  if (e != hipSuccess) return e;
  const dim3 grid_x(group_grid((a.nrb_max + 1) / 2, a.vl.n_seqs, a.n_heads));
  { KernelTimer kt_("k_block_extract", st); hipLaunchKernelGGL((k_block_extract<D>), grid_x, dim3(512), lds_x, st, a); }
  return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs& a, int d, hipStream_t st) {
  if (a.n_heads == 0 || a.vl.n_seqs == 0 || a.nrb_max == 0) {
    return hipSuccess;
  }
  return d == 64 ? compress_impl<64>(a, st) : compress_impl<128>(a, st);
}

}  // namespace cma
