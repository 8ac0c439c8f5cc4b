// Argument blocks and launchers shared between the C ABI layer and the kernels.
#pragma once
#include "common.hpp"

namespace cma {

// Brackets one kernel launch with HIP events when timing is enabled.
struct KernelTimer {
  KernelTimer(const char* name, hipStream_t st);
  ~KernelTimer();
  const char* name;
  hipStream_t st;
  void* ev0;
};

struct AttnMapsArgs {
  const uint16_t* q;  // bf16 inputs
  const uint16_t* k;
  const float* qf;    // fp32 inputs
  const float* kf;
  Varlen vl;
  const float* scale;
  const float* bias;
  void* maps;
  int64_t head_stride;
  int32_t n_heads;
  bool in_bf16, out_bf16, packed;
  int32_t rows_cap;  // single-row path: keys its LDS holds (set by the launcher)
  int32_t n_rb;      // block-row slots per (sequence, head) (set by the launcher)
};
hipError_t launch_attn_maps(const AttnMapsArgs& a, int d, int max_q, int max_k, hipStream_t st);

struct CosineArgs {
  const void* recv;
  const void* send;
  bool bf16;
  int32_t n_batch, n_recv, n_send;
  int64_t len, rh, rb, sh, sb;
  float* cos;
  int32_t* argmax;
  float* margin;
  float* part;   // [splits][n_batch][n_recv][n_send]
  float* rnorm;  // [splits][n_batch][n_recv]
  float* snorm;  // [splits][n_batch][n_send]
  int32_t splits;
  int64_t kchunk;
};
struct CosinePlan {
  int32_t splits;
  int64_t kchunk;
  size_t ws_bytes;
};
CosinePlan plan_cosine(int32_t n_batch, int32_t n_recv, int32_t n_send, int64_t len, bool bf16);
hipError_t launch_cosine(const CosineArgs& a, hipStream_t st);

// Fused head mapping: receiver maps scored inside the Gram producer (never stored).
struct FusedMapArgs {
  const uint16_t* q;  // receiver queries / keys [n_recv, total, 128] bf16
  const uint16_t* k;
  Varlen vl;          // one problem per sequence (square: nq == nk)
  const float* scale;
  const float* bias;
  const uint16_t* send;  // sender maps, dense bf16, as cma_attn_maps writes them
  int64_t send_hs;       // elements per sender head
  int32_t n_recv, n_send;
  int32_t n_qt;          // query tiles of 32 rows of the longest sequence (the split count)
  CosineArgs fin;        // finalize: part / rnorm / snorm with splits = n_qt, outputs
};
constexpr int kFusedRows = 32;    // query rows per workgroup (one split)
constexpr int kFusedHeads = 32;   // receiver heads per workgroup
constexpr int kFusedSend = 384;   // senders per workgroup (up to twelve 32-wide tiles)
constexpr int kFusedMaxLen = 4096;  // longest mapped prefix
size_t fused_map_ws_bytes(int32_t n_batch, int32_t n_recv, int32_t n_send, int32_t max_seqlen);
hipError_t launch_head_map_fused(const FusedMapArgs& a, hipStream_t st);

struct CompressArgs {
  const uint16_t* q;
  const uint16_t* k;
  Varlen vl;
  const float* scale;
  const float* bias;
  float tau;
  int32_t n_heads, n_block_rows;
  int32_t nrb_max;  // block-rows of the longest query sequence (grid)
  int32_t ncb_max;  // key blocks of the longest key sequence (<= kMaxBlockRows)
  int32_t* row_ptr;
  int32_t* col_idx;
  uint16_t* vals;
  int64_t capacity;
  int32_t* nnz;
  float* block_mass;
  float* row_stats;
  // workspace
  int32_t* counts;     // [n_heads * n_block_rows]
  uint32_t* kept;      // [n_heads * n_block_rows * kWords]
  float* lse2;         // [n_heads * total_q] log2-domain log-sum-exp per query row
};
constexpr int kMaxBlockRows = 256;  // sequences up to 16384 tokens
constexpr int kMaxVPages = 65536;   // pages of a paged V head (byte offsets stay below 2^31)
constexpr int kWords = kMaxBlockRows / 32;
size_t compress_ws_bytes(int32_t n_heads, int32_t n_block_rows, int64_t total_q);
hipError_t launch_compress(const CompressArgs& a, int d, hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t st);

struct MappedAvArgs {
  // dense source
  const void* maps;
  bool maps_bf16, packed;
  int64_t head_stride;
  // bsr source
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const uint16_t* vals;
  int32_t n_block_rows;
  const int32_t* row_end;  // block-row g's blocks end at row_end[g] (NULL: row_ptr[g + 1])
  int32_t n_key_blocks;    // tiled V blocks per head: sum over sequences of ceil(nk / 64)
  // paged V: vt is the page pool [n_v][v_n_pages][64 * 128]; key block c of
  // sequence s is page v_pages[s * v_page_stride + c]
  const int32_t* v_pages;
  int32_t v_page_stride, v_n_pages;
  int32_t n_send, n_recv, d;
  int32_t n_v, v_group;  // V heads; receiver head h reads V head h / v_group
  const float* M;
  int64_t M_stride;
  const void* v;
  bool v_bf16;
  bool v_key_major;  // v is [n_v][d][total_k] (else [n_v][total_k][d])
  bool v_tiled;      // v is in the fused kernel's operand order (bsr path)
  Varlen vl;
  void* out;
  bool out_bf16;
  uint16_t* vt;  // bsr path: tiled V [n_v][n_key_blocks][64 * d] (v itself or the workspace), or the page pool
  int32_t max_q, max_k;  // longest query / key sequence (host maxima)
  // indexed path (one sender per receiver head): sender[s * sender_stride + h]
  const int32_t* sender;
  int64_t sender_stride;
  int32_t* plan_roff;   // [2 n_seqs]: first block-row of each sequence, then its first key block
  int32_t* plan_order;  // [n_seqs * n_recv]: receiver heads of each sequence, ordered by sender
  int32_t* plan_pairs;  // [plan_cap]: (sequence << 7 | pair) of every work item, -1 past the end
  int64_t plan_cap;
  // dense path: partial rows of split rows (workspace; NULL: rows are not split)
  float* part;
  size_t part_bytes;
  // block-sparse path: this launch's senders are send0 .. send0 + n_send - 1 of
  // m_ld (the row length of M); accum adds the result to out instead of storing it
  int32_t send0, m_ld;
  bool accum;
};
constexpr int kDenseSplitMax = 8;  // workgroups per row of a dense launch of few rows
hipError_t launch_mapped_av_dense(const MappedAvArgs& a, hipStream_t st);
hipError_t launch_mapped_av_bsr(const MappedAvArgs& a, hipStream_t st);
hipError_t launch_mapped_av_indexed(const MappedAvArgs& a, hipStream_t st);
hipError_t launch_tile_v(const MappedAvArgs& a, hipStream_t st);  // v -> vt (bf16, d = 128)
int cu_count();  // compute units of the current device (cached per device)
hipError_t launch_onehot(const int32_t* argmax, int32_t n_batch, int32_t n_recv, int32_t n_send,
                         float* M, hipStream_t st);

}  // namespace cma
