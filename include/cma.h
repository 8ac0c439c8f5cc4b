/*
 * cma.h -- C ABI of the MI355X (gfx950) library for cross-model reuse of causal
 * attention probability maps.
 *
 * Sources (web pages; sections named after their own headings):
 *  [IAM]     "IAM: Efficient Inference through Attention Mapping between
 *            Different-scale LLMs", paper notes (ACL 2025): Method 1 (cosine of
 *            flattened maps), Method 2 (mapped-layer order), Method 4 (per-head
 *            argmax at prefill; decode reuses the small model's attention rows).
 *  [MapFlow] news article on "Accelerating Cross-Model LLM Inference via
 *            Attention Map Reuse": approach section (receiver heads are learned
 *            linear combinations of sender head maps; receiver keeps its own V),
 *            storage-and-execution section (block-sparse retention of regular
 *            2-D blocks by cumulative probability, two phases -- block
 *            statistics, then extraction -- without the dense map; fused kernel
 *            that mixes heads on chip and multiplies by V).
 *  [GLIDE]   "GLIDE: Guided Layerwise Hybrid Attention", sections II-A/II-B
 *            (causal scaled dot-product softmax attention).
 *
 * Conventions for every call
 *  - Pointers are DEVICE pointers unless marked [host]. The caller allocates and
 *    owns all memory; the library never allocates, frees or keeps pointers.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and the
 *    call returns before it completes. The return value reports argument
 *    validation (done before any HIP call) and launch errors only; faults
 *    surface at the caller's next synchronisation.
 *  - Errors: CMA_OK (0) or a negative status; cma_last_error() gives a message
 *    (thread-local). Nothing is launched when validation fails.
 *  - Layout: head-major [H, T, d] row-major tensors. Several sequences are
 *    packed along T and described by cma_varlen. Query row i of a sequence with
 *    nq query rows and nk keys sits at key position nk - nq + i (bottom-right
 *    alignment) and sees keys 0 .. nk - nq + i.
 *  - Results are deterministic: identical inputs give bitwise identical outputs
 *    (no floating-point atomics in reductions).
 *  - bf16 is stored as 16-bit bit patterns (uint16); conversions from fp32 round
 *    to nearest even.
 */
#ifndef CMA_H
#define CMA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CMA_OK 0
#define CMA_EINVAL (-1)       /* NULL required pointer, bad sizes, inconsistent arguments */
#define CMA_EUNSUPPORTED (-2) /* head dim, dtype or layout combination not built */
#define CMA_ENOSPC (-3)       /* workspace smaller than the size the call requires */
#define CMA_EHIP (-4)         /* a HIP launch or runtime call failed */

typedef enum { CMA_F32 = 0, CMA_BF16 = 1 } cma_dtype;

/* Map storage. DENSE: each (head, sequence) map is nq x nk row-major. PACKED:
 * only the visible entries, row by row; row i holds nk - nq + i + 1 entries and
 * starts at i*(nk - nq) + i*(i+1)/2 (for a square map: i(i+1)/2 + j). Per head,
 * the sequences' maps follow each other in sequence order; head h starts at
 * h * head_stride elements. */
typedef enum { CMA_MAP_DENSE = 0, CMA_MAP_PACKED = 1 } cma_map_layout;

/* Packed variable-length sequences.
 * cu_seqlens_q/k: [n_seqs + 1] int32 start rows of each sequence in the query
 *   (Q, output) and key (K, V) tensors; nondecreasing.
 * seqused_q/k: optional [n_seqs] rows actually used per sequence (defaults to
 *   the cu_seqlens spacing); lets a sequence use a prefix of its reserved rows.
 * max_seqlen_q/k [host]: upper bounds of the used lengths (grid sizing).
 * total_q/k [host]: rows of the query / key tensors (bounds for validation;
 *   rows beyond them are never touched). */
typedef struct {
  int32_t n_seqs;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  const int32_t* seqused_q;
  const int32_t* seqused_k;
  int32_t max_seqlen_q;
  int32_t max_seqlen_k;
  int64_t total_q;
  int64_t total_k;
} cma_varlen;

/* Per-kernel timing (profiling aid). While enabled, every kernel the library
 * launches is bracketed by two HIP events recorded on the launch's own stream.
 * cma_timing_collect() waits for the recorded events (host-blocking) and adds
 * their elapsed times to per-kernel totals; cma_timing_get() reads a kernel's
 * total milliseconds and launch count by name (see cma_timing_name()); reset
 * clears everything. Thread-safe; disabled by default (then no events exist). */
int cma_timing_enable(int on);
int cma_timing_collect(void);
double cma_timing_get(const char* kernel, int64_t* launches);
const char* cma_timing_name(int index); /* NULL past the last kernel seen */
void cma_timing_reset(void);

/* Library version (major*10000 + minor*100 + patch). */
int cma_version(void);
/* Message for the last non-OK status returned on this thread. */
const char* cma_last_error(void);

/* Elements per head of a map buffer for the given host-side sequence lengths
 * ([host] arrays of n_seqs); -1 on invalid arguments. */
int64_t cma_maps_elems(int32_t n_seqs, const int32_t* len_q, const int32_t* len_k,
                       cma_map_layout layout);

/*
 * cma_attn_maps -- causal attention probability maps per head ([GLIDE] II-B;
 * materialised explicitly as [IAM] Method 4 requires).
 *   A_ij = softmax_j( logit_scale[h] * <q_i, k_j> + key0_bias[h] * [j == 0] )
 * over the visible keys j; invisible entries are 0 (DENSE) or absent (PACKED).
 * q [n_heads, total_q, d], k [n_heads, total_k, d] in `in_dt` (bf16 or f32);
 * logit_scale [n_heads] (beta_h / sqrt(d)); key0_bias [n_heads] or NULL (0);
 * maps: n_heads * head_stride elements of `out_dt`; head_stride >=
 * cma_maps_elems(...). d must be 64 or 128. Each sequence needs nq <= nk.
 * Returns EINVAL for bad pointers/sizes, EUNSUPPORTED for other d.
 */
int cma_attn_maps(const void* q, const void* k, cma_dtype in_dt, int32_t n_heads, int32_t d,
                  const cma_varlen* vl, const float* logit_scale, const float* key0_bias,
                  void* maps, cma_dtype out_dt, cma_map_layout layout, int64_t head_stride,
                  void* stream);

/*
 * cma_head_map_cosine -- head mapping by cosine similarity of flattened maps
 * ([IAM] Methods 1 and 4). For each problem b of n_batch:
 *   cos[b,h,j] = <R_bh, S_bj> / (|R_bh| |S_bj|)   (0 if a norm is 0)
 *   argmax[b,h] = the j with the largest cos (lowest j on ties)
 *   margin[b,h] = largest minus second-largest cos (+inf if n_send == 1)
 * R_bh = recv + b*recv_bstride + h*recv_hstride, S_bj likewise, each `len`
 * elements of `dt` (bf16 or f32). Strides are in elements and must be
 * multiples of 8; pointers 16-byte aligned. cos [n_batch, n_recv, n_send] and
 * margin [n_batch, n_recv] may be NULL; argmax [n_batch, n_recv] is required.
 * Computed as a split-K Gram product with fp32 accumulation, reduced in a fixed
 * order. Needs `workspace` of cma_head_map_cosine_workspace(...) bytes.
 */
size_t cma_head_map_cosine_workspace(int32_t n_batch, int32_t n_recv, int32_t n_send, int64_t len,
                                     cma_dtype dt);
int cma_head_map_cosine(const void* recv, const void* send, cma_dtype dt, int32_t n_batch,
                        int32_t n_recv, int32_t n_send, int64_t len, int64_t recv_hstride,
                        int64_t recv_bstride, int64_t send_hstride, int64_t send_bstride,
                        float* cos, int32_t* argmax, float* margin, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * cma_head_map_fused -- the head mapping of cma_head_map_cosine without storing the
 * receivers' maps ([IAM] Methods 1 and 4; the maps must be explicit softmax
 * outputs, which is why the pages rule out a flash-style kernel, so here they
 * are formed tile by tile on chip and consumed by the Gram product at once).
 * One problem per sequence b of `vl` (square: nq == nk, max_seqlen <= 4096):
 *   R_bh = the causal map of receiver head h on sequence b, computed from
 *          recv_q / recv_k [n_recv, total, d] bf16 with recv_scale / recv_bias
 *          [n_recv] as in cma_attn_maps, each value rounded to bf16 (the values a
 *          stored map would hold);
 *   S_bj = sender head j's map of sequence b as stored by cma_attn_maps with
 *          CMA_MAP_DENSE, bf16: send_maps + j * send_head_stride, sequence b at the
 *          sum of n_u^2 over earlier sequences (rows starting on 16 bytes are read
 *          16 bytes at a time, others element by element);
 * cos [n_seqs, n_recv, n_send] (or NULL), argmax [n_seqs, n_recv], margin (or
 * NULL) as cma_head_map_cosine defines them (the zeros above the diagonal add
 * nothing, so the value equals the cosine of the flattened causal entries).
 * d = 128. Workspace: cma_head_map_fused_workspace(n_seqs, n_recv, n_send,
 * max_seqlen) bytes (per 32-row split, the partial Gram and norms).
 */
size_t cma_head_map_fused_workspace(int32_t n_batch, int32_t n_recv, int32_t n_send, int32_t max_seqlen);
int cma_head_map_fused(const void* recv_q, const void* recv_k, int32_t n_recv, int32_t d, const float* recv_scale,
                       const float* recv_bias, const void* send_maps, int64_t send_head_stride, int32_t n_send,
                       const cma_varlen* vl, float* cos, int32_t* argmax, float* margin, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * cma_block_compress -- two-phase block-sparse compression of causal maps
 * ([MapFlow] storage and execution), never forming the dense map.
 * Phase 1 sweeps QK^T once per block-row with an online softmax and keeps, per
 * 64x64 block (r, c <= r), its probability mass; per block-row the masses are
 * normalised by their sum, ordered largest first (ties: lower column) and the
 * shortest prefix whose running sum reaches `tau` is kept (tau >= 1 keeps all).
 * Phase 2 recomputes only the kept blocks and writes them as bf16.
 * Sequence s has nq = used query rows and nk = used key rows (keys at rows
 * cu_seqlens_k[s] ..). nq = nk is a whole prompt; nq < nk is a prefill chunk
 * ([MapFlow] storage and execution, closing paragraph: chunked prefill): the
 * nq queries are the last nq positions of the nk-token sequence (bottom-right
 * alignment). Blocks are laid out per sequence from its first token, so nk - nq
 * must be a multiple of 64: block-row r of the chunk is block-row kb0 + r of
 * the sequence (kb0 = (nk - nq) / 64) and has blocks 0 .. kb0 + r; it equals
 * that block-row of the whole prompt's compression. A sequence that breaks this
 * rule gets no output rows (CMA_CHECK_LENGTHS=1 turns it into CMA_EINVAL). Edge
 * blocks are zero-padded.
 * Outputs (block-sparse row format, BSR):
 *   row_ptr [n_heads * n_block_rows + 1] int32, n_block_rows = sum_s ceil(nq_s/64);
 *     global block-row g = h * n_block_rows + (block-rows of earlier sequences) + r;
 *   col_idx [capacity] int32, kept block columns (sequence-local), ascending per row;
 *   vals [capacity, 64, 64] bf16 blocks, zeros above the diagonal, each stored as
 *     four panels of 16 columns: element (i, j) of a block is at
 *     (j / 16) * 1024 + i * 16 + j % 16 (a 16-column slice of consecutive rows
 *     is contiguous, which is how the fused pass reads it);
 *   nnz [1] int32: number of kept blocks. If nnz > capacity nothing is written to
 *     col_idx / vals (row_ptr and nnz still are): allocate nnz and call again.
 *     cma_bsr_capacity() is always enough.
 *   block_mass (optional) [n_heads, sum_s (R_s kb0_s + R_s(R_s+1)/2)] fp32 masses,
 *     R_s = ceil(nq_s/64); block-row r of sequence s holds kb0_s + r + 1 masses from
 *     offset_s + r kb0_s + r(r+1)/2 (packed lower-triangular for whole prompts);
 *   row_stats (optional) [n_heads, total_q, 2] fp32 (row max of the logits,
 *     sum of exp(logit - max)) at each query row.
 * Requires d in {64, 128}, max_seqlen_q and max_seqlen_k <= 16384, tau > 0. Workspace:
 * cma_block_compress_workspace(...) bytes.
 */
int64_t cma_bsr_max_blocks(int32_t n_heads, int32_t n_seqs, const int32_t* len_host);
/* Blocks a compression can keep at most, prefill chunks included: n_heads * sum_s
 * (R_s kb0_s + R_s(R_s+1)/2), R_s = ceil(nq_s/64), kb0_s = (nk_s - nq_s) / 64
 * (len_q, len_k [host]; len_k NULL: whole prompts, as cma_bsr_max_blocks); -1 on
 * bad arguments. */
int64_t cma_bsr_capacity(int32_t n_heads, int32_t n_seqs, const int32_t* len_q, const int32_t* len_k);
size_t cma_block_compress_workspace(int32_t n_heads, int32_t n_block_rows, int32_t max_seqlen,
                                    int64_t total_q);
int cma_block_compress(const void* q, const void* k, cma_dtype in_dt, int32_t n_heads, int32_t d,
                       const cma_varlen* vl, const float* logit_scale, const float* key0_bias,
                       float tau, int32_t n_block_rows, int32_t* row_ptr, int32_t* col_idx,
                       void* vals, int64_t capacity, int32_t* nnz, float* block_mass,
                       float* row_stats, void* workspace, size_t workspace_bytes, void* stream);

/*
 * cma_block_compress_noalloc -- cma_block_compress for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments, results and kernels, without the
 * workspace. Its scratch (per-block-row counts, kept-column masks and per-query
 * log-sum-exp: cma_block_compress_workspace(...) bytes) lives in one static
 * device array of CMA_NOALLOC_SCRATCH_BYTES per GPU, part of the library's code
 * object. Returns CMA_ENOSPC (nothing launched) when the call needs more; calls
 * no hipMalloc, hipFree or allocating routine. Every call on one GPU uses that
 * GPU's one array: calls that overlap on a GPU (other streams, other threads)
 * race and must be serialised by the caller. The first call on a device takes
 * the array's device address (hipGetSymbolAddress) and keeps it.
 */
#define CMA_NOALLOC_SCRATCH_BYTES (16u << 20)
int cma_block_compress_noalloc(const void* q, const void* k, cma_dtype in_dt, int32_t n_heads, int32_t d,
                               const cma_varlen* vl, const float* logit_scale, const float* key0_bias, float tau,
                               int32_t n_block_rows, int32_t* row_ptr, int32_t* col_idx, void* vals,
                               int64_t capacity, int32_t* nnz, float* block_mass, float* row_stats, void* stream);

/* Layout of the receiver's V. TOKEN_MAJOR: [n_recv, total_k, d] (row t holds the
 * d values of key t). KEY_MAJOR: [n_recv, d, total_k] (row e holds feature e of
 * every key). TILED (block-sparse source, bf16, d = 128 only): the fused
 * kernel's operand order, [n_recv, n_key_blocks, 64 * 128]: sequence s's nk_s
 * keys in 64-key blocks, its first block at the sum of ceil(nk/64) over earlier
 * sequences (n_key_blocks = that sum over all sequences; for whole prompts the
 * same numbering as the block-sparse maps' block-rows); within block c, element
 *   ((ks * 4 + dt) * 64 + L) * 8 + e  =  V[key 64c + 16ks + 8(L/32) + e][feature 32dt + L%32]
 * for ks, dt in 0..3, L in 0..63, e in 0..7, zero past the sequence end. A V
 * projection can write it directly; cma_mapped_av builds it from the other two
 * layouts in its workspace.
 * PAGED (block-sparse source, bf16, d = 128): V in a paged cache ([MapFlow]
 * storage and execution, closing paragraph: PagedAttention): the `v` argument
 * then points to a cma_paged_v descriptor in HOST memory. Each page holds one
 * 64-key block of one V head in the TILED block order; the page table maps key
 * block c of sequence s to a page. */
typedef enum { CMA_V_TOKEN_MAJOR = 0, CMA_V_KEY_MAJOR = 1, CMA_V_TILED = 2, CMA_V_PAGED = 3 } cma_v_layout;

/* Paged V (CMA_V_PAGED). pages: device [n_v_heads, n_pages, 64 * 128] bf16,
 * 16-byte aligned (page p of V head g at (g * n_pages + p) * 8192 elements);
 * page_table: device int32, key block c of sequence s in page
 * page_table[s * page_stride + c] (c < ceil(nk_s / 64) <= page_stride), every
 * entry in [0, n_pages); 1 <= n_pages <= 65536. Keys past a sequence's end
 * inside its last page must be zero (cma_tile_v_paged writes them so). */
typedef struct {
  const void* pages;
  const int32_t* page_table;
  int32_t page_stride;
  int32_t n_pages;
} cma_paged_v;

/*
 * cma_tile_v -- V in the TILED layout (see cma_v_layout) from TOKEN_MAJOR or
 * KEY_MAJOR V, bf16, d = 128: what cma_mapped_av does in its workspace, as a call of
 * its own, so that a caller can tile V once (e.g. on another stream, or for several
 * calls) and pass CMA_V_TILED. v: n_v_heads heads; vt [n_v_heads, n_block_rows,
 * 64 * 128] bf16 (device, 16-byte aligned), every block of every sequence written
 * (zeros past the sequence's end); n_block_rows = sum_s ceil(len_s / 64) as for the block-sparse maps.
 * The varlen's used query lengths are the sequence lengths (square sequences).
 */
int cma_tile_v(const void* v, cma_v_layout v_layout, int32_t n_v_heads, int32_t d, const cma_varlen* vl,
               int32_t n_block_rows, void* vt, void* stream);

/*
 * cma_tile_v_paged -- as cma_tile_v, into the pages of a paged V cache: key
 * block c of sequence s (its nk_s used keys) goes to page
 * dst->page_table[s * dst->page_stride + c] of every V head (zeros past the
 * sequence's end); pages the table does not name are left as they are. dst is a
 * host descriptor whose `pages` the call writes. Returns EINVAL for a bad
 * descriptor (the table's entries are trusted to lie in [0, n_pages)).
 */
int cma_tile_v_paged(const void* v, cma_v_layout v_layout, int32_t n_v_heads, int32_t d, const cma_varlen* vl,
                     const cma_paged_v* dst, void* stream);

/* Where cma_mapped_av reads the sender maps from. */
typedef enum { CMA_SRC_DENSE = 0, CMA_SRC_BSR = 1 } cma_src_kind;
typedef struct {
  cma_src_kind kind;
  /* CMA_SRC_DENSE: maps as written by cma_attn_maps (any nq <= nk, incl. decode rows) */
  const void* maps;
  cma_dtype maps_dt;
  cma_map_layout layout;
  int64_t head_stride;
  /* CMA_SRC_BSR: output of cma_block_compress (whole prompts or prefill chunks).
   * Block-row g's blocks are entries row_ptr[g] .. row_end[g] - 1 of col_idx and
   * vals; row_end = NULL means row_ptr[g + 1] (the packed form cma_block_compress
   * writes). With row_end, rows may sit anywhere in (and share) a pool of blocks,
   * e.g. block-rows looked up in a prefix cache (cma_prefix_index_*) next to
   * freshly compressed ones. */
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const void* vals;
  int32_t n_block_rows;
  const int32_t* row_end;
  /* key blocks of all sequences, sum_s ceil(nk_s / 64) (the TILED V's block
   * count); 0 means n_block_rows (whole prompts) */
  int32_t n_key_blocks;
} cma_maps_src;

/*
 * cma_mapped_av -- fused mapped attention x V ([MapFlow] approach and fused
 * kernel; [IAM] Method 4 decode with a one-hot M):
 *   O_h = ( sum_j M[s][h][j] * A_j ) @ V_{h / g}     for every sequence s,
 * where A_j is sender head j's map as stored (zeros off the kept blocks for a
 * BSR source) and g = n_recv / n_v_heads receiver heads share one V head
 * (grouped V; n_v_heads = n_recv: one V per receiver head). The mixed map is
 * formed on chip and never written to memory.
 * M: fp32 [*, n_recv, n_send], sequence s uses M + s * M_seq_stride
 * (M_seq_stride = 0: one matrix for all). v (n_v_heads heads) in `v_layout` (see
 * cma_v_layout, with n_v_heads in place of n_recv) and out [n_recv, total_q, d]
 * in v_dt / out_dt (bf16 or f32); accumulation is fp32. n_v_heads >= 1 must
 * divide n_recv. d in {64, 128}, 1 <= n_send <= 64. A BSR source with more than
 * 32 senders runs one pass per group of 32 (later passes add into `out`, so bf16
 * output is rounded once per group). A BSR
 * source needs bf16 V and d = 128; its sequences are whole prompts or prefill
 * chunks as in cma_block_compress (out holds the chunk's nq rows; V its nk keys,
 * nk <= 16384); with TOKEN_MAJOR or KEY_MAJOR V it first writes the TILED copy
 * of V into `workspace` (cma_mapped_av_workspace(...) bytes: n_v_heads *
 * n_key_blocks * 64 * d * 2), with TILED or PAGED V it needs no workspace and
 * launches only the fused pass. A dense source takes TOKEN_MAJOR or KEY_MAJOR V and
 * needs no workspace; given one of cma_mapped_av_workspace(...) bytes (2 MiB for
 * 256 CUs at d = 128), a launch of fewer rows than twice the CUs (a long-context
 * decode of a small batch) splits each row's keys over up to 8 workgroups and
 * adds the partial rows in a fixed order (deterministic; the sums may differ in
 * the last bits from an unsplit launch).
 */
size_t cma_mapped_av_workspace(const cma_maps_src* src, int32_t n_v_heads, int32_t d, int64_t total_k,
                               cma_v_layout v_layout);
int cma_mapped_av(const cma_maps_src* src, int32_t n_send, const float* M, int64_t M_seq_stride,
                  int32_t n_recv, int32_t n_v_heads, const void* v, cma_dtype v_dt, cma_v_layout v_layout,
                  int32_t d, const cma_varlen* vl, void* out, cma_dtype out_dt, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * cma_mapped_av_indexed -- mapped attention x V with one sender per receiver head,
 * the head map of [IAM] Methods 1 and 4 (each receiver head reuses the map of its
 * most similar sender head):
 *   O_h = A_{sender[s][h]} @ V_{h / g}          for every sequence s,
 * the same result as cma_mapped_av with the one-hot M of cma_onehot_mix, without
 * reading the other senders' maps. sender: int32 [*, n_recv] (device), sequence s
 * uses sender + s * sender_seq_stride (0: one row for all sequences), e.g. the
 * argmax of cma_head_map_cosine; an index outside [0, n_send) gives zero rows.
 * Source: BSR only (output of cma_block_compress; whole prompts or prefill
 * chunks, optional row_end); V bf16, d = 128, any cma_v_layout (n_v_heads
 * heads, n_v_heads >= 1 dividing n_recv); out [n_recv, total_q, 128] bf16 or
 * f32, fp32 accumulation. n_recv <= 256, 1 <= n_send <= 256, max_seqlen_q and
 * max_seqlen_k <= 16384, n_seqs < 2^24. Each receiver head reads only its
 * sender's kept blocks. Workspace (device, 16-byte aligned):
 * cma_mapped_av_indexed_workspace(...) bytes, which hold the tiled copy of V
 * (unless v_layout is TILED or PAGED), each sequence's block-row and key-block
 * offsets, the heads ordered by sender per sequence and the work-item table;
 * n_block_rows must equal sum_s ceil(nq_s / 64), as for every BSR call.
 */
size_t cma_mapped_av_indexed_workspace(const cma_maps_src* src, int32_t n_recv, int32_t n_v_heads, int32_t d,
                                       int32_t n_seqs, cma_v_layout v_layout);
int cma_mapped_av_indexed(const cma_maps_src* src, int32_t n_send, const int32_t* sender,
                          int64_t sender_seq_stride, int32_t n_recv, int32_t n_v_heads, const void* v,
                          cma_dtype v_dt, cma_v_layout v_layout, int32_t d, const cma_varlen* vl, void* out,
                          cma_dtype out_dt, void* workspace, size_t workspace_bytes, void* stream);

/*
 * cma_onehot_mix -- IAM head map as a mixing matrix ([IAM] Method 4):
 * M[b][h][j] = (j == argmax[b][h]) for argmax [n_batch, n_recv] (device);
 * M [n_batch, n_recv, n_send] fp32 (device). Indices outside [0, n_send) give
 * an all-zero row.
 */
int cma_onehot_mix(const int32_t* argmax, int32_t n_batch, int32_t n_recv, int32_t n_send,
                   float* M, void* stream);

/*
 * cma_mapped_layers -- receiver layers to map for a ratio ([IAM] Method 2):
 * from the last layer down to layer round(0.8 L), then from layer round(0.2 L)
 * upwards; the first round(0.2 L) layers are never mapped. Writes up to `cap`
 * 0-indexed layers in priority order to out [host]; returns the count
 * (round-half-up(ratio * L), clamped to the available layers) or a negative
 * status.
 */
int cma_mapped_layers(int32_t n_layers, double ratio, int32_t* out, int32_t cap);

/*
 * cma_mapping_plan -- the tau_e / tau_t thresholds of [IAM] Method 4 for a batch
 * of n requests [host]. A prompt shorter than tau_e is first extended by ordinary
 * generation to tau_e tokens, and only then is the head map built; the
 * similarity is computed on the first tau_t tokens of a longer context:
 *   gen_before[i] = max(0, tau_e - prompt_len[i])
 *   sim_len[i]    = min(prompt_len[i] + gen_before[i], tau_t)
 * prompt_len, gen_before, sim_len: [n] int32, host memory owned by the caller.
 * Returns CMA_OK, or CMA_EINVAL (nothing written) for n < 0, a null array with
 * n > 0, a negative prompt length, tau_e < 0 or tau_t < 1.
 */
int cma_mapping_plan(int32_t n, const int32_t* prompt_len, int32_t tau_e, int32_t tau_t,
                     int32_t* gen_before, int32_t* sim_len);

/*
 * Prefix-hash index of compressed sender states ([MapFlow] storage and execution,
 * second component: the sender's block-sparse rows differ in number per layer and
 * position; a prefix-hash index that carries the preceding context lets a
 * receiver find the cached blocks it can reuse, and one sender state serves
 * several downstream models). Host memory only; the block pool it points into
 * (col_idx / vals of a block-sparse source) is the caller's.
 *
 * cma_prefix_hashes: chained hashes of the n_tokens / 64 whole 64-token blocks of
 * a token sequence [host]: hash b = FNV-1a-64 over (hash b-1 as 8 little-endian
 * bytes; `seed` for b = 0) followed by tokens 64b .. 64b + 63 (4 little-endian
 * bytes each). Equal hashes b mean equal tokens 0 .. 64b + 63 (up to 64-bit
 * collisions), i.e. the same causal context for block-row b. `seed` names what
 * else the rows depend on (sender model and layer weights).
 * cma_fnv1a64: the plain FNV-1a-64 of a byte string.
 *
 * cma_prefix_index_create(n_heads, capacity): an empty index of at most
 * `capacity` entries, each holding n_heads (begin, count) pairs; NULL on bad
 * arguments or allocation failure. destroy frees it.
 * insert(layer, hash, begin[n_heads], count[n_heads]): caches one block-row (for
 * every sender head, its blocks begin[h] .. begin[h] + count[h] - 1 of the pool);
 * re-inserting a key replaces its entry; CMA_ENOSPC when full (evict first),
 * CMA_EINVAL for a negative begin or count.
 * lookup(layer, hashes[n], begin[n][n_heads], count[n][n_heads]): the number of
 * leading hashes found (a request reuses block-rows 0 .. hits - 1), their entries
 * copied out (begin / count may be NULL); refreshes their recency.
 * erase: 1 if the key was present, 0 if not. evict_lru: removes the least
 * recently used entry and returns 1 with its key and pairs (the caller frees that
 * pool space), 0 if empty. size: entries held. All calls are thread-safe; a
 * negative return is a status.
 */
typedef struct cma_prefix_index cma_prefix_index;
int cma_prefix_hashes(const int32_t* tokens, int64_t n_tokens, uint64_t seed, uint64_t* hashes);
uint64_t cma_fnv1a64(const void* data, size_t n_bytes);
cma_prefix_index* cma_prefix_index_create(int32_t n_heads, int64_t capacity);
void cma_prefix_index_destroy(cma_prefix_index* index);
int cma_prefix_index_insert(cma_prefix_index* index, int32_t layer, uint64_t hash, const int32_t* begin,
                            const int32_t* count);
int64_t cma_prefix_index_lookup(cma_prefix_index* index, int32_t layer, const uint64_t* hashes, int64_t n,
                                int32_t* begin, int32_t* count);
int cma_prefix_index_erase(cma_prefix_index* index, int32_t layer, uint64_t hash);
int cma_prefix_index_evict_lru(cma_prefix_index* index, int32_t* layer, uint64_t* hash, int32_t* begin,
                               int32_t* count);
int64_t cma_prefix_index_size(cma_prefix_index* index);

#ifdef __cplusplus
}
#endif
#endif /* CMA_H */
