// C ABI: argument validation (before any HIP call), workspace sizing, dispatch.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"

using namespace cma;

// ------------------------------------------------------------------ kernel timing
namespace {
struct PendingTiming {
  std::string name;
  hipEvent_t a, b;
};
struct TimingState {
  std::mutex mu;
  std::vector<hipEvent_t> pool;
  std::vector<PendingTiming> pending;
  std::map<std::string, std::pair<double, int64_t>> totals;
  std::vector<std::string> names;
};
std::atomic<bool> g_timing{false};
TimingState& timing() {
  static TimingState* t = new TimingState();  // lives for the process
  return *t;
}
hipEvent_t take_event() {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

namespace cma {
KernelTimer::KernelTimer(const char* n, hipStream_t s) : name(n), st(s), ev0(nullptr) {
  if (!g_timing.load(std::memory_order_relaxed)) return;
  hipEvent_t e = take_event();
  if (e && hipEventRecord(e, st) == hipSuccess) ev0 = e;
}
KernelTimer::~KernelTimer() {
  if (!ev0) return;
  hipEvent_t e1 = take_event();
  if (!e1 || hipEventRecord(e1, st) != hipSuccess) return;
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.pending.push_back({name, static_cast<hipEvent_t>(ev0), e1});
}
}  // namespace cma

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CMA_EHIP, "%s: %s", what, hipGetErrorString(e));
  static const bool sync_debug = [] {
    const char* s = getenv("CMA_SYNC_DEBUG");
    return s && s[0] == '1';
  }();
  if (sync_debug) {
    hipError_t e2 = hipDeviceSynchronize();
    if (e2 != hipSuccess) return fail(CMA_EHIP, "%s (sync): %s", what, hipGetErrorString(e2));
  }
  return CMA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// CMA_CHECK_LENGTHS=1: every call copies the device sequence tables to the host
// (synchronously) and checks them against the host maxima and tensor sizes.
bool check_lengths_enabled() {
  static const bool on = [] {
    const char* s = getenv("CMA_CHECK_LENGTHS");
    return s && s[0] == '1';
  }();
  return on;
}

int check_lengths_on_device(const cma_varlen* vl, bool need_k, bool chunks) {
  const int n = vl->n_seqs;
  if (n == 0) return CMA_OK;
  std::vector<int32_t> cq(n + 1), ck(n + 1), uq, uk;
  auto get = [&](const int32_t* p, std::vector<int32_t>& v, size_t cnt) {
    v.resize(cnt);
    return hipMemcpy(v.data(), p, cnt * sizeof(int32_t), hipMemcpyDeviceToHost);
  };
  if (get(vl->cu_seqlens_q, cq, n + 1) != hipSuccess) return fail(CMA_EHIP, "copying cu_seqlens_q failed");
  const int32_t* cuk = vl->cu_seqlens_k ? vl->cu_seqlens_k : vl->cu_seqlens_q;
  if (get(cuk, ck, n + 1) != hipSuccess) return fail(CMA_EHIP, "copying cu_seqlens_k failed");
  if (vl->seqused_q && get(vl->seqused_q, uq, n) != hipSuccess) return fail(CMA_EHIP, "copying seqused_q failed");
  if (vl->seqused_k && get(vl->seqused_k, uk, n) != hipSuccess) return fail(CMA_EHIP, "copying seqused_k failed");
  const int64_t tk = vl->cu_seqlens_k ? vl->total_k : vl->total_q;
  for (int s = 0; s < n; ++s) {
    const int64_t lq = vl->seqused_q ? uq[s] : (int64_t)cq[s + 1] - cq[s];
    const int64_t lk = vl->seqused_k ? uk[s] : (int64_t)ck[s + 1] - ck[s];
    if (cq[s] < 0 || ck[s] < 0 || cq[s + 1] < cq[s] || ck[s + 1] < ck[s])
      return fail(CMA_EINVAL, "cu_seqlens must be nonnegative and nondecreasing (sequence %d)", s);
    if (lq < 0 || lk < 0 || cq[s] + lq > vl->total_q || (need_k && ck[s] + lk > tk))
      return fail(CMA_EINVAL, "sequence %d runs past the tensor rows", s);
    if (lq > vl->max_seqlen_q || (need_k && lk > vl->max_seqlen_k))
      return fail(CMA_EINVAL, "sequence %d is longer (%lld / %lld) than max_seqlen_q / _k (%d / %d)", s,
                  (long long)lq, (long long)lk, vl->max_seqlen_q, vl->max_seqlen_k);
    if (chunks && (lk < lq || (lk - lq) % kBlock))
      return fail(CMA_EINVAL, "sequence %d: a block-sparse query chunk needs nk >= nq with nk - nq a multiple of %d",
                  s, kBlock);
  }
  return CMA_OK;
}

// chunks: block-sparse calls, whose sequences are whole prompts or prefill chunks
// (nk >= nq, nk - nq a multiple of 64).
int check_varlen(const cma_varlen* vl, bool need_k, bool chunks = false) {
  if (!vl) return fail(CMA_EINVAL, "varlen descriptor is NULL");
  if (vl->n_seqs < 0) return fail(CMA_EINVAL, "n_seqs < 0");
  if (vl->n_seqs > 0 && (!vl->cu_seqlens_q || (need_k && !vl->cu_seqlens_k)))
    return fail(CMA_EINVAL, "cu_seqlens pointer is NULL");
  if (vl->max_seqlen_q < 0 || vl->max_seqlen_k < 0) return fail(CMA_EINVAL, "negative max_seqlen");
  if (vl->total_q < 0 || vl->total_k < 0) return fail(CMA_EINVAL, "negative total rows");
  if (vl->max_seqlen_q > vl->total_q || (need_k && vl->max_seqlen_k > vl->total_k))
    return fail(CMA_EINVAL, "max_seqlen exceeds the tensor rows");
  if (check_lengths_enabled()) return check_lengths_on_device(vl, need_k, chunks);
  return CMA_OK;
}

Varlen to_varlen(const cma_varlen* vl) {
  Varlen v;
  v.n_seqs = vl->n_seqs;
  v.cu_q = vl->cu_seqlens_q;
  v.cu_k = vl->cu_seqlens_k ? vl->cu_seqlens_k : vl->cu_seqlens_q;
  v.used_q = vl->seqused_q;
  v.used_k = vl->seqused_k;
  v.total_q = vl->total_q;
  v.total_k = vl->cu_seqlens_k ? vl->total_k : vl->total_q;
  return v;
}

bool dtype_ok(cma_dtype d) { return d == CMA_F32 || d == CMA_BF16; }

}  // namespace

extern "C" {

int cma_timing_enable(int on) {
  g_timing.store(on != 0);
  return CMA_OK;
}

int cma_timing_collect(void) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  for (auto& p : t.pending) {
    if (hipEventSynchronize(p.b) != hipSuccess) return fail(CMA_EHIP, "event synchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) return fail(CMA_EHIP, "elapsed time failed");
    auto it = t.totals.find(p.name);
    if (it == t.totals.end()) {
      t.names.push_back(p.name);
      it = t.totals.emplace(p.name, std::make_pair(0.0, (int64_t)0)).first;
    }
    it->second.first += ms;
    it->second.second += 1;
    t.pool.push_back(p.a);
    t.pool.push_back(p.b);
  }
  t.pending.clear();
  return CMA_OK;
}

double cma_timing_get(const char* kernel, int64_t* launches) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  auto it = kernel ? t.totals.find(kernel) : t.totals.end();
  if (it == t.totals.end()) {
    if (launches) *launches = 0;
    return 0.0;
  }
  if (launches) *launches = it->second.second;
  return it->second.first;
}

const char* cma_timing_name(int index) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  if (index < 0 || index >= (int)t.names.size()) return nullptr;
  return t.names[index].c_str();
}

void cma_timing_reset(void) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.totals.clear();
  t.names.clear();
}

int cma_version(void) { return 100; }

const char* cma_last_error(void) { return g_err; }

int64_t cma_maps_elems(int32_t n_seqs, const int32_t* len_q, const int32_t* len_k,
                       cma_map_layout layout) {
  if (n_seqs < 0 || (n_seqs > 0 && (!len_q || !len_k))) return -1;
  int64_t tot = 0;
  for (int s = 0; s < n_seqs; ++s) {
    const int64_t nq = len_q[s], nk = len_k[s];
    if (nq < 0 || nk < nq) return -1;
    tot += layout == CMA_MAP_PACKED ? nq * (nk - nq) + nq * (nq + 1) / 2 : nq * nk;
  }
  return tot;
}

int cma_attn_maps(const void* q, const void* k, cma_dtype in_dt, int32_t n_heads, int32_t d,
                  const cma_varlen* vl, const float* logit_scale, const float* key0_bias,
                  void* maps, cma_dtype out_dt, cma_map_layout layout, int64_t head_stride,
                  void* stream) {
  if (int e = check_varlen(vl, true)) return e;
  if (n_heads < 0) return fail(CMA_EINVAL, "n_heads < 0");
  if (!dtype_ok(in_dt) || !dtype_ok(out_dt)) return fail(CMA_EINVAL, "bad dtype");
  if (layout != CMA_MAP_DENSE && layout != CMA_MAP_PACKED) return fail(CMA_EINVAL, "bad layout");
  if (n_heads == 0 || vl->n_seqs == 0) return CMA_OK;
  if (!q || !k || !logit_scale || !maps) return fail(CMA_EINVAL, "NULL q, k, logit_scale or maps");
  if (head_stride < 0) return fail(CMA_EINVAL, "negative head_stride");
  if (in_dt == CMA_BF16) {
    if (d != 64 && d != 128) return fail(CMA_EUNSUPPORTED, "bf16 attn_maps supports d = 64 or 128 (got %d)", d);
    if (!aligned16(q) || !aligned16(k)) return fail(CMA_EINVAL, "q and k must be 16-byte aligned");
  } else if (d < 1 || d > 256) {
    return fail(CMA_EUNSUPPORTED, "fp32 attn_maps supports 1 <= d <= 256 (got %d)", d);
  }
  AttnMapsArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.qf = static_cast<const float*>(q);
  a.kf = static_cast<const float*>(k);
  a.vl = to_varlen(vl);
  a.scale = logit_scale;
  a.bias = key0_bias;
  a.maps = maps;
  a.head_stride = head_stride;
  a.n_heads = n_heads;
  a.in_bf16 = in_dt == CMA_BF16;
  a.out_bf16 = out_dt == CMA_BF16;
  a.packed = layout == CMA_MAP_PACKED;
  return hip_status(launch_attn_maps(a, d, vl->max_seqlen_q, vl->max_seqlen_k, static_cast<hipStream_t>(stream)),
                    "attn_maps launch");
}

size_t cma_head_map_cosine_workspace(int32_t n_batch, int32_t n_recv, int32_t n_send, int64_t len,
                                     cma_dtype dt) {
  if (n_batch <= 0 || n_recv <= 0 || n_send <= 0 || len <= 0) return 0;
  return plan_cosine(n_batch, n_recv, n_send, len, dt == CMA_BF16).ws_bytes;
}

int cma_head_map_cosine(const void* recv, const void* send, cma_dtype dt, int32_t n_batch,
                        int32_t n_recv, int32_t n_send, int64_t len, int64_t recv_hstride,
                        int64_t recv_bstride, int64_t send_hstride, int64_t send_bstride,
                        float* cos, int32_t* argmax, float* margin, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dt)) return fail(CMA_EINVAL, "bad dtype");
  if (n_batch < 0 || n_recv < 0 || n_send < 0 || len < 0) return fail(CMA_EINVAL, "negative size");
  if (n_batch == 0 || n_recv == 0) return CMA_OK;
  if (n_send == 0) return fail(CMA_EINVAL, "n_send must be positive");
  if (n_send > 384) return fail(CMA_EUNSUPPORTED, "n_send > 384");
  if (len == 0) return fail(CMA_EINVAL, "len must be positive");
  if (!recv || !send || !argmax) return fail(CMA_EINVAL, "NULL recv, send or argmax");
  if (recv_hstride < 0 || recv_bstride < 0 || send_hstride < 0 || send_bstride < 0)
    return fail(CMA_EINVAL, "negative stride");
  if (dt == CMA_BF16) {
    if (!aligned16(recv) || !aligned16(send)) return fail(CMA_EINVAL, "recv/send must be 16-byte aligned");
    if ((recv_hstride | recv_bstride | send_hstride | send_bstride) % 8)
      return fail(CMA_EINVAL, "bf16 strides must be multiples of 8 elements");
  }
  const CosinePlan pl = plan_cosine(n_batch, n_recv, n_send, len, dt == CMA_BF16);
  if (!workspace || workspace_bytes < pl.ws_bytes)
    return fail(CMA_ENOSPC, "workspace of %zu bytes needed", pl.ws_bytes);
  CosineArgs a{};
  a.recv = recv;
  a.send = send;
  a.bf16 = dt == CMA_BF16;
  a.n_batch = n_batch;
  a.n_recv = n_recv;
  a.n_send = n_send;
  a.len = len;
  a.rh = recv_hstride;
  a.rb = recv_bstride;
  a.sh = send_hstride;
  a.sb = send_bstride;
  a.cos = cos;
  a.argmax = argmax;
  a.margin = margin;
  float* ws = static_cast<float*>(workspace);
  a.part = ws;
  a.rnorm = a.part + (size_t)pl.splits * n_batch * n_recv * n_send;
  a.snorm = a.rnorm + (size_t)pl.splits * n_batch * n_recv;
  a.splits = pl.splits;
  a.kchunk = pl.kchunk;
  return hip_status(launch_cosine(a, static_cast<hipStream_t>(stream)), "head_map_cosine launch");
}

int64_t cma_bsr_max_blocks(int32_t n_heads, int32_t n_seqs, const int32_t* len_host) {
  if (n_heads < 0 || n_seqs < 0 || (n_seqs > 0 && !len_host)) return -1;
  int64_t tot = 0;
  for (int s = 0; s < n_seqs; ++s) {
    if (len_host[s] < 0) return -1;
    const int64_t R = (len_host[s] + kBlock - 1) / kBlock;
    tot += R * (R + 1) / 2;
  }
  return tot * n_heads;
}

size_t cma_head_map_fused_workspace(int32_t n_batch, int32_t n_recv, int32_t n_send, int32_t max_seqlen) {
  if (n_batch <= 0 || n_recv <= 0 || n_send <= 0 || max_seqlen <= 0) return 0;
  return fused_map_ws_bytes(n_batch, n_recv, n_send, max_seqlen);
}

int cma_head_map_fused(const void* recv_q, const void* recv_k, int32_t n_recv, int32_t d, const float* recv_scale,
                       const float* recv_bias, const void* send_maps, int64_t send_head_stride, int32_t n_send,
                       const cma_varlen* vl, float* cos, int32_t* argmax, float* margin, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (int e = check_varlen(vl, true)) return e;
  if (n_recv < 0 || n_send < 0 || send_head_stride < 0) return fail(CMA_EINVAL, "negative size");
  if (d != 128) return fail(CMA_EUNSUPPORTED, "head_map_fused supports d = 128 (got %d)", d);
  if (n_recv == 0 || vl->n_seqs == 0) return CMA_OK;
  if (n_send == 0) return fail(CMA_EINVAL, "n_send must be positive");
  if (vl->max_seqlen_q != vl->max_seqlen_k)
    return fail(CMA_EINVAL, "head_map_fused maps square sequences (max_seqlen_q == max_seqlen_k)");
  if (vl->max_seqlen_q > kFusedMaxLen) return fail(CMA_EUNSUPPORTED, "head_map_fused supports sequences up to %d", kFusedMaxLen);
  if (!recv_q || !recv_k || !recv_scale || !send_maps || !argmax)
    return fail(CMA_EINVAL, "NULL recv_q, recv_k, recv_scale, send_maps or argmax");
  if (!aligned16(recv_q) || !aligned16(recv_k) || !aligned16(send_maps))
    return fail(CMA_EINVAL, "recv_q, recv_k and send_maps must be 16-byte aligned");
  const size_t need = fused_map_ws_bytes(vl->n_seqs, n_recv, n_send, vl->max_seqlen_q);
  if (!workspace || workspace_bytes < need) return fail(CMA_ENOSPC, "workspace of %zu bytes needed", need);
  FusedMapArgs a{};
  a.q = static_cast<const uint16_t*>(recv_q);
  a.k = static_cast<const uint16_t*>(recv_k);
  a.vl = to_varlen(vl);
  a.scale = recv_scale;
  a.bias = recv_bias;
  a.send = static_cast<const uint16_t*>(send_maps);
  a.send_hs = send_head_stride;
  a.n_recv = n_recv;
  a.n_send = n_send;
  a.n_qt = (vl->max_seqlen_q + kFusedRows - 1) / kFusedRows;
  a.fin.bf16 = true;
  a.fin.n_batch = vl->n_seqs;
  a.fin.n_recv = n_recv;
  a.fin.n_send = n_send;
  a.fin.cos = cos;
  a.fin.argmax = argmax;
  a.fin.margin = margin;
  float* ws = static_cast<float*>(workspace);
  a.fin.part = ws;
  a.fin.rnorm = a.fin.part + (size_t)a.n_qt * vl->n_seqs * n_recv * n_send;
  a.fin.snorm = a.fin.rnorm + (size_t)a.n_qt * vl->n_seqs * n_recv;
  a.fin.splits = a.n_qt;
  return hip_status(launch_head_map_fused(a, static_cast<hipStream_t>(stream)), "head_map_fused launch");
}

int64_t cma_bsr_capacity(int32_t n_heads, int32_t n_seqs, const int32_t* len_q, const int32_t* len_k) {
  if (n_heads < 0 || n_seqs < 0 || (n_seqs > 0 && !len_q)) return -1;
  int64_t tot = 0;
  for (int s = 0; s < n_seqs; ++s) {
    const int64_t nq = len_q[s], nk = len_k ? len_k[s] : len_q[s];
    if (nq < 0 || nk < nq) return -1;
    const int64_t R = (nq + kBlock - 1) / kBlock, kb0 = (nk - nq) / kBlock;
    tot += R * kb0 + R * (R + 1) / 2;
  }
  return tot * n_heads;
}

size_t cma_block_compress_workspace(int32_t n_heads, int32_t n_block_rows, int32_t max_seqlen,
                                    int64_t total_q) {
  (void)max_seqlen;
  if (n_heads < 0 || n_block_rows < 0 || total_q < 0) return 0;
  return compress_ws_bytes(n_heads, n_block_rows, total_q);
}

}  // extern "C"

// Scratch of the allocation-free compression entry point: one array per GPU the
// library runs on (part of the library's code object, held until the process
// ends). Host code never passes the array's name to a kernel: on the host it is
// a stand-in, not a device address. The device address is taken once per device
// with hipGetSymbolAddress (that device current) and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[CMA_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(CMA_EHIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(CMA_EUNSUPPORTED, "device index %d beyond 63", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(CMA_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CMA_OK;
}

int block_compress_impl(const void* q, const void* k, cma_dtype in_dt, int32_t n_heads, int32_t d,
                        const cma_varlen* vl, const float* logit_scale, const float* key0_bias, float tau,
                        int32_t n_block_rows, int32_t* row_ptr, int32_t* col_idx, void* vals, int64_t capacity,
                        int32_t* nnz, float* block_mass, float* row_stats, void* workspace, size_t workspace_bytes,
                        void* stream, bool static_scratch);
}  // namespace

extern "C" {

int cma_block_compress(const void* q, const void* k, cma_dtype in_dt, int32_t n_heads, int32_t d,
                       const cma_varlen* vl, const float* logit_scale, const float* key0_bias,
                       float tau, int32_t n_block_rows, int32_t* row_ptr, int32_t* col_idx,
                       void* vals, int64_t capacity, int32_t* nnz, float* block_mass,
                       float* row_stats, void* workspace, size_t workspace_bytes, void* stream) {
  return block_compress_impl(q, k, in_dt, n_heads, d, vl, logit_scale, key0_bias, tau, n_block_rows, row_ptr,
                             col_idx, vals, capacity, nnz, block_mass, row_stats, workspace, workspace_bytes, stream,
                             false);
}

int cma_block_compress_noalloc(const void* q, const void* k, cma_dtype in_dt, int32_t n_heads, int32_t d,
                               const cma_varlen* vl, const float* logit_scale, const float* key0_bias, float tau,
                               int32_t n_block_rows, int32_t* row_ptr, int32_t* col_idx, void* vals,
                               int64_t capacity, int32_t* nnz, float* block_mass, float* row_stats, void* stream) {
  return block_compress_impl(q, k, in_dt, n_heads, d, vl, logit_scale, key0_bias, tau, n_block_rows, row_ptr,
                             col_idx, vals, capacity, nnz, block_mass, row_stats, nullptr, 0, stream, true);
}

}  // extern "C"

namespace {
int block_compress_impl(const void* q, const void* k, cma_dtype in_dt, int32_t n_heads, int32_t d,
                        const cma_varlen* vl, const float* logit_scale, const float* key0_bias, float tau,
                        int32_t n_block_rows, int32_t* row_ptr, int32_t* col_idx, void* vals, int64_t capacity,
                        int32_t* nnz, float* block_mass, float* row_stats, void* workspace, size_t workspace_bytes,
                        void* stream, bool static_scratch) {
  if (int e = check_varlen(vl, true, true)) return e;
  if (in_dt != CMA_BF16) return fail(CMA_EUNSUPPORTED, "block_compress needs bf16 q and k");
  if (d != 64 && d != 128) return fail(CMA_EUNSUPPORTED, "block_compress supports d = 64 or 128 (got %d)", d);
  if (!(tau > 0.0f) || std::isnan(tau)) return fail(CMA_EINVAL, "tau must be > 0");
  if (n_heads < 0 || n_block_rows < 0 || capacity < 0) return fail(CMA_EINVAL, "negative size");
  if (vl->max_seqlen_q > kMaxBlockRows * kBlock || vl->max_seqlen_k > kMaxBlockRows * kBlock)
    return fail(CMA_EUNSUPPORTED, "sequences (queries and keys) are limited to %d tokens", kMaxBlockRows * kBlock);
  if (!row_ptr || !nnz) return fail(CMA_EINVAL, "NULL row_ptr or nnz");
  if (capacity > 0 && (!col_idx || !vals)) return fail(CMA_EINVAL, "NULL col_idx or vals");
  if (vals && !aligned16(vals)) return fail(CMA_EINVAL, "vals must be 16-byte aligned");
  if (n_heads > 0 && vl->n_seqs > 0) {
    if (!q || !k || !logit_scale) return fail(CMA_EINVAL, "NULL q, k or logit_scale");
    if (!aligned16(q) || !aligned16(k)) return fail(CMA_EINVAL, "q and k must be 16-byte aligned");
  }
  const size_t need = compress_ws_bytes(n_heads, n_block_rows, vl->total_q);
  if (static_scratch) {
    if (need > (size_t)CMA_NOALLOC_SCRATCH_BYTES)
      return fail(CMA_ENOSPC, "the call needs %zu bytes of scratch; the static scratch holds %zu", need,
                  (size_t)CMA_NOALLOC_SCRATCH_BYTES);
    if (int e = scratch_address(&workspace)) return e;
    workspace_bytes = CMA_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace || workspace_bytes < need) return fail(CMA_ENOSPC, "workspace of %zu bytes needed", need);
  CompressArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.vl = to_varlen(vl);
  a.scale = logit_scale;
  a.bias = key0_bias;
  a.tau = tau;
  a.n_heads = n_heads;
  a.n_block_rows = n_block_rows;
  a.nrb_max = (vl->max_seqlen_q + kBlock - 1) / kBlock;
  a.ncb_max = (std::max(vl->max_seqlen_q, vl->max_seqlen_k) + kBlock - 1) / kBlock;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.vals = static_cast<uint16_t*>(vals);
  a.capacity = capacity;
  a.nnz = nnz;
  a.block_mass = block_mass;
  a.row_stats = row_stats;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* w = static_cast<char*>(workspace);
  const size_t g = (size_t)n_heads * n_block_rows;
  a.counts = reinterpret_cast<int32_t*>(w);
  w += al(g * sizeof(int32_t));
  a.kept = reinterpret_cast<uint32_t*>(w);
  w += al(g * kWords * sizeof(uint32_t));
  a.lse2 = reinterpret_cast<float*>(w);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (n_heads == 0 || vl->n_seqs == 0 || a.nrb_max == 0) {
    // nothing to compress: row_ptr = 0, nnz = 0 (a fill kernel, safe under graph capture)
    hipError_t e = launch_fill_i32(row_ptr, (int64_t)n_heads * n_block_rows + 1, 0, st);
    if (e == hipSuccess) e = launch_fill_i32(nnz, 1, 0, st);
    return hip_status(e, "block_compress (empty)");
  }
  if (static_scratch) {
    // the shared scratch keeps the previous call's counts: clear them (a fill
    // kernel) so that a block-row this call does not reach cannot inherit one
    hipError_t e = launch_fill_i32(a.counts, (int64_t)n_heads * n_block_rows, 0, st);
    if (e != hipSuccess) return hip_status(e, "block_compress_noalloc (clear)");
  }
  return hip_status(launch_compress(a, d, st), "block_compress launch");
}
}  // namespace

extern "C" {

}  // extern "C"

namespace {
int32_t key_blocks_of(const cma_maps_src* src) { return src->n_key_blocks > 0 ? src->n_key_blocks : src->n_block_rows; }

// Checks shared by the block-sparse passes, and the source and V fields of `a`.
// Needs a.n_v and a.vl set. For TOKEN_MAJOR / KEY_MAJOR V the tiled copy goes to
// the workspace at `vt_ws` (the caller checks its size).
int setup_bsr(MappedAvArgs& a, const cma_maps_src* src, const void* v, cma_v_layout v_layout, const cma_varlen* vl,
              uint16_t* vt_ws) {
  if (!src->row_ptr || !src->col_idx || !src->vals) return fail(CMA_EINVAL, "NULL block-sparse arrays");
  if (vl->max_seqlen_q > kMaxBlockRows * kBlock || vl->max_seqlen_k > kMaxBlockRows * kBlock)
    return fail(CMA_EUNSUPPORTED, "block-sparse passes support sequences up to %d tokens", kMaxBlockRows * kBlock);
  if (!aligned16(src->vals)) return fail(CMA_EINVAL, "vals must be 16-byte aligned");
  if (src->n_block_rows < 0 || src->n_key_blocks < 0) return fail(CMA_EINVAL, "negative n_block_rows or n_key_blocks");
  if (vl->max_seqlen_q > 0 && src->n_block_rows == 0)
    return fail(CMA_EINVAL, "n_block_rows must cover the sequences' 64-row blocks");
  if (vl->max_seqlen_q > vl->max_seqlen_k)
    return fail(CMA_EINVAL, "block-sparse sequences have at least as many keys as queries (max_seqlen_q > max_seqlen_k)");
  a.row_ptr = src->row_ptr;
  a.row_end = src->row_end;
  a.col_idx = src->col_idx;
  a.vals = static_cast<const uint16_t*>(src->vals);
  a.n_block_rows = src->n_block_rows;
  a.n_key_blocks = key_blocks_of(src);
  a.v_key_major = v_layout == CMA_V_KEY_MAJOR;
  if (v_layout == CMA_V_PAGED) {
    const cma_paged_v* pv = static_cast<const cma_paged_v*>(v);
    if (!pv->pages || !pv->page_table) return fail(CMA_EINVAL, "NULL pages or page_table in the paged V");
    if (!aligned16(pv->pages)) return fail(CMA_EINVAL, "V pages must be 16-byte aligned");
    if (pv->n_pages < 1 || pv->n_pages > kMaxVPages)
      return fail(CMA_EUNSUPPORTED, "paged V supports 1 .. %d pages", kMaxVPages);
    if ((int64_t)pv->page_stride * kBlock < vl->max_seqlen_k)
      return fail(CMA_EINVAL, "page_stride (%d) holds fewer key blocks than the longest sequence", pv->page_stride);
    a.vt = const_cast<uint16_t*>(static_cast<const uint16_t*>(pv->pages));
    a.v_pages = pv->page_table;
    a.v_page_stride = pv->page_stride;
    a.v_n_pages = pv->n_pages;
    a.v_tiled = true;
  } else if (v_layout == CMA_V_TILED) {
    if (!aligned16(v)) return fail(CMA_EINVAL, "tiled V must be 16-byte aligned");
    a.vt = const_cast<uint16_t*>(static_cast<const uint16_t*>(v));
    a.v_tiled = true;
  } else {
    if (!a.v_key_major && !aligned16(v)) return fail(CMA_EINVAL, "token-major V must be 16-byte aligned");
    a.vt = vt_ws;
  }
  return CMA_OK;
}

bool v_layout_ok(cma_v_layout l) {
  return l == CMA_V_TOKEN_MAJOR || l == CMA_V_KEY_MAJOR || l == CMA_V_TILED || l == CMA_V_PAGED;
}
size_t tiled_v_bytes(const cma_maps_src* src, int32_t n_v_heads, int32_t d) {
  return (size_t)n_v_heads * key_blocks_of(src) * kBlock * d * sizeof(uint16_t);
}
}  // namespace

extern "C" {

size_t cma_mapped_av_workspace(const cma_maps_src* src, int32_t n_v_heads, int32_t d, int64_t total_k,
                               cma_v_layout v_layout) {
  (void)total_k;
  if (!src || n_v_heads <= 0 || d <= 0) return 0;
  // dense: partial rows of a launch of fewer rows than twice the CUs, split
  // kDenseSplitMax ways at most
  if (src->kind == CMA_SRC_DENSE) return (size_t)kDenseSplitMax * 2 * cu_count() * d * sizeof(float);
  if (src->kind != CMA_SRC_BSR || v_layout == CMA_V_TILED || v_layout == CMA_V_PAGED || src->n_block_rows <= 0)
    return 0;
  return tiled_v_bytes(src, n_v_heads, d);
}

int cma_mapped_av(const cma_maps_src* src, int32_t n_send, const float* M, int64_t M_seq_stride,
                  int32_t n_recv, int32_t n_v_heads, const void* v, cma_dtype v_dt, cma_v_layout v_layout,
                  int32_t d, const cma_varlen* vl, void* out, cma_dtype out_dt, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (!src) return fail(CMA_EINVAL, "NULL maps source");
  if (!v_layout_ok(v_layout)) return fail(CMA_EINVAL, "bad V layout");
  if (int e = check_varlen(vl, true, src->kind == CMA_SRC_BSR)) return e;
  if (!dtype_ok(v_dt) || !dtype_ok(out_dt)) return fail(CMA_EINVAL, "bad dtype");
  if (n_send < 0 || n_recv < 0 || M_seq_stride < 0) return fail(CMA_EINVAL, "negative size");
  if (n_v_heads < 1 || (n_recv > 0 && n_recv % n_v_heads != 0))
    return fail(CMA_EINVAL, "n_v_heads (%d) must be >= 1 and divide n_recv (%d)", n_v_heads, n_recv);
  if (d != 64 && d != 128) return fail(CMA_EUNSUPPORTED, "mapped_av supports d = 64 or 128 (got %d)", d);
  if (n_recv == 0 || vl->n_seqs == 0) return CMA_OK;
  if (n_send == 0 || n_send > 64) return fail(CMA_EUNSUPPORTED, "mapped_av supports 1 <= n_send <= 64");
  if (!M || !v || !out) return fail(CMA_EINVAL, "NULL M, v or out");
  MappedAvArgs a{};
  a.n_send = n_send;
  a.n_recv = n_recv;
  a.n_v = n_v_heads;
  a.v_group = n_recv / n_v_heads;
  a.d = d;
  a.M = M;
  a.M_stride = M_seq_stride;
  a.v = v;
  a.v_bf16 = v_dt == CMA_BF16;
  a.v_key_major = v_layout == CMA_V_KEY_MAJOR;
  a.v_tiled = v_layout == CMA_V_TILED;
  a.vl = to_varlen(vl);
  a.out = out;
  a.out_bf16 = out_dt == CMA_BF16;
  a.max_q = vl->max_seqlen_q;
  a.max_k = vl->max_seqlen_k;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (src->kind == CMA_SRC_DENSE) {
    if (!src->maps) return fail(CMA_EINVAL, "NULL maps");
    if (!dtype_ok(src->maps_dt)) return fail(CMA_EINVAL, "bad maps dtype");
    if (src->layout != CMA_MAP_DENSE && src->layout != CMA_MAP_PACKED) return fail(CMA_EINVAL, "bad layout");
    if (src->head_stride < 0) return fail(CMA_EINVAL, "negative head_stride");
    a.maps = src->maps;
    a.maps_bf16 = src->maps_dt == CMA_BF16;
    a.packed = src->layout == CMA_MAP_PACKED;
    a.head_stride = src->head_stride;
    if (a.v_tiled || v_layout == CMA_V_PAGED)
      return fail(CMA_EUNSUPPORTED, "tiled and paged V serve block-sparse sources only");
    if (workspace) {  // optional: room to split the rows of a launch of few rows
      if (!aligned16(workspace)) return fail(CMA_EINVAL, "workspace must be 16-byte aligned");
      a.part = static_cast<float*>(workspace);
      a.part_bytes = workspace_bytes;
    }
    return hip_status(launch_mapped_av_dense(a, st), "mapped_av (dense) launch");
  }
  if (src->kind != CMA_SRC_BSR) return fail(CMA_EINVAL, "bad source kind");
  if (v_dt != CMA_BF16 || d != 128) return fail(CMA_EUNSUPPORTED, "block-sparse mapped_av needs bf16 V and d = 128");
  const bool tiles = v_layout == CMA_V_TOKEN_MAJOR || v_layout == CMA_V_KEY_MAJOR;
  if (tiles) {
    const size_t need = tiled_v_bytes(src, n_v_heads, d);
    if (!workspace || workspace_bytes < need) return fail(CMA_ENOSPC, "workspace of %zu bytes needed", need);
    if (!aligned16(workspace)) return fail(CMA_EINVAL, "workspace must be 16-byte aligned");
  }
  if (int e = setup_bsr(a, src, v, v_layout, vl, static_cast<uint16_t*>(workspace))) return e;
  return hip_status(launch_mapped_av_bsr(a, st), "mapped_av (block-sparse) launch");
}

namespace {
int tile_v_common(const void* v, cma_v_layout v_layout, int32_t n_v_heads, int32_t d, const cma_varlen* vl,
                  int32_t n_key_blocks, void* vt, const cma_paged_v* pv, void* stream) {
  if (v_layout != CMA_V_TOKEN_MAJOR && v_layout != CMA_V_KEY_MAJOR)
    return fail(CMA_EINVAL, "tile_v reads token-major or key-major V");
  if (int e = check_varlen(vl, true)) return e;
  if (n_v_heads < 0 || n_key_blocks < 0) return fail(CMA_EINVAL, "negative size");
  if (d != 128) return fail(CMA_EUNSUPPORTED, "tile_v supports d = 128");
  if (n_v_heads == 0 || vl->n_seqs == 0 || vl->max_seqlen_k == 0) return CMA_OK;
  if (vl->max_seqlen_k > kMaxBlockRows * kBlock)
    return fail(CMA_EUNSUPPORTED, "tile_v supports sequences up to %d tokens", kMaxBlockRows * kBlock);
  if (!pv && n_key_blocks == 0) return fail(CMA_EINVAL, "n_block_rows must cover the sequences' 64-key blocks");
  if (!v || !vt) return fail(CMA_EINVAL, "NULL v or destination");
  if (!aligned16(vt) || (v_layout == CMA_V_TOKEN_MAJOR && !aligned16(v)))
    return fail(CMA_EINVAL, "v (token-major) and the destination must be 16-byte aligned");
  MappedAvArgs a{};
  a.n_v = n_v_heads;
  a.d = d;
  a.v = v;
  a.v_bf16 = true;
  a.v_key_major = v_layout == CMA_V_KEY_MAJOR;
  a.vl = to_varlen(vl);
  a.vt = static_cast<uint16_t*>(vt);
  a.n_key_blocks = n_key_blocks;
  a.max_q = vl->max_seqlen_q;
  a.max_k = vl->max_seqlen_k;
  if (pv) {
    if (!pv->page_table) return fail(CMA_EINVAL, "NULL page_table");
    if (pv->n_pages < 1 || pv->n_pages > kMaxVPages)
      return fail(CMA_EUNSUPPORTED, "paged V supports 1 .. %d pages", kMaxVPages);
    if ((int64_t)pv->page_stride * kBlock < vl->max_seqlen_k)
      return fail(CMA_EINVAL, "page_stride (%d) holds fewer key blocks than the longest sequence", pv->page_stride);
    a.v_pages = pv->page_table;
    a.v_page_stride = pv->page_stride;
    a.v_n_pages = pv->n_pages;
  }
  return hip_status(launch_tile_v(a, static_cast<hipStream_t>(stream)), "tile_v launch");
}
}  // namespace

int cma_tile_v(const void* v, cma_v_layout v_layout, int32_t n_v_heads, int32_t d, const cma_varlen* vl,
               int32_t n_block_rows, void* vt, void* stream) {
  return tile_v_common(v, v_layout, n_v_heads, d, vl, n_block_rows, vt, nullptr, stream);
}

int cma_tile_v_paged(const void* v, cma_v_layout v_layout, int32_t n_v_heads, int32_t d, const cma_varlen* vl,
                     const cma_paged_v* dst, void* stream) {
  if (!dst) return fail(CMA_EINVAL, "NULL paged V descriptor");
  return tile_v_common(v, v_layout, n_v_heads, d, vl, 0, const_cast<void*>(dst->pages), dst, stream);
}

// Workspace of the indexed path: [tiled V (unless V is tiled or paged)][block-row
// and key-block offsets][order][pairs], each part on a 256-byte boundary. The
// pair table holds at most sum_s ceil(R_s / 2) <= (n_block_rows + n_seqs) / 2 items.
}  // extern "C"
namespace {
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
struct IdxLayout {  // byte offsets into the workspace; the tiled V (if any) starts at 0
  size_t roff, order, pairs, total;
  int64_t cap;
};
IdxLayout idx_layout(const cma_maps_src* src, int32_t n_recv, int32_t n_v_heads, int32_t d, int32_t n_seqs,
                     bool own_v) {
  IdxLayout l{};
  l.cap = ((int64_t)src->n_block_rows + n_seqs) / 2 + 1;
  l.roff = own_v ? round256(tiled_v_bytes(src, n_v_heads, d)) : 0;
  l.order = l.roff + round256((size_t)2 * n_seqs * sizeof(int32_t));
  l.pairs = l.order + round256((size_t)n_seqs * n_recv * sizeof(int32_t));
  l.total = l.pairs + round256((size_t)l.cap * sizeof(int32_t));
  return l;
}
}  // namespace
extern "C" {

size_t cma_mapped_av_indexed_workspace(const cma_maps_src* src, int32_t n_recv, int32_t n_v_heads, int32_t d,
                                       int32_t n_seqs, cma_v_layout v_layout) {
  if (!src || src->kind != CMA_SRC_BSR || n_recv <= 0 || n_v_heads <= 0 || d <= 0 || n_seqs <= 0 ||
      src->n_block_rows < 0 || src->n_key_blocks < 0)
    return 0;
  const bool own_v = v_layout == CMA_V_TOKEN_MAJOR || v_layout == CMA_V_KEY_MAJOR;
  return idx_layout(src, n_recv, n_v_heads, d, n_seqs, own_v).total;
}

int cma_mapped_av_indexed(const cma_maps_src* src, int32_t n_send, const int32_t* sender,
                          int64_t sender_seq_stride, int32_t n_recv, int32_t n_v_heads, const void* v,
                          cma_dtype v_dt, cma_v_layout v_layout, int32_t d, const cma_varlen* vl, void* out,
                          cma_dtype out_dt, void* workspace, size_t workspace_bytes, void* stream) {
  if (!src) return fail(CMA_EINVAL, "NULL maps source");
  if (src->kind != CMA_SRC_BSR) return fail(CMA_EUNSUPPORTED, "mapped_av_indexed reads block-sparse maps only");
  if (!v_layout_ok(v_layout)) return fail(CMA_EINVAL, "bad V layout");
  if (int e = check_varlen(vl, true, true)) return e;
  if (!dtype_ok(v_dt) || !dtype_ok(out_dt)) return fail(CMA_EINVAL, "bad dtype");
  if (n_send < 0 || n_recv < 0 || sender_seq_stride < 0) return fail(CMA_EINVAL, "negative size");
  if (n_v_heads < 1 || (n_recv > 0 && n_recv % n_v_heads != 0))
    return fail(CMA_EINVAL, "n_v_heads (%d) must be >= 1 and divide n_recv (%d)", n_v_heads, n_recv);
  if (n_recv == 0 || vl->n_seqs == 0) return CMA_OK;
  if (v_dt != CMA_BF16 || d != 128) return fail(CMA_EUNSUPPORTED, "mapped_av_indexed needs bf16 V and d = 128");
  if (n_send < 1 || n_send > 256) return fail(CMA_EUNSUPPORTED, "mapped_av_indexed supports 1 <= n_send <= 256");
  if (n_recv > 256) return fail(CMA_EUNSUPPORTED, "mapped_av_indexed supports n_recv <= 256");
  if (vl->n_seqs >= (1 << 24)) return fail(CMA_EUNSUPPORTED, "mapped_av_indexed supports fewer than 2^24 sequences");
  if (!sender || !v || !out) return fail(CMA_EINVAL, "NULL sender, v or out");
  const bool own_v = v_layout == CMA_V_TOKEN_MAJOR || v_layout == CMA_V_KEY_MAJOR;
  const IdxLayout l = idx_layout(src, n_recv, n_v_heads, d, vl->n_seqs, own_v);
  if (!workspace || workspace_bytes < l.total) return fail(CMA_ENOSPC, "workspace of %zu bytes needed", l.total);
  if (!aligned16(workspace)) return fail(CMA_EINVAL, "workspace must be 16-byte aligned");
  MappedAvArgs a{};
  a.n_send = n_send;
  a.n_recv = n_recv;
  a.n_v = n_v_heads;
  a.v_group = n_recv / n_v_heads;
  a.d = d;
  a.v = v;
  a.v_bf16 = true;
  a.vl = to_varlen(vl);
  a.out = out;
  a.out_bf16 = out_dt == CMA_BF16;
  a.max_q = vl->max_seqlen_q;
  a.max_k = vl->max_seqlen_k;
  char* ws = static_cast<char*>(workspace);
  if (int e = setup_bsr(a, src, v, v_layout, vl, reinterpret_cast<uint16_t*>(ws))) return e;
  a.sender = sender;
  a.sender_stride = sender_seq_stride;
  a.plan_roff = reinterpret_cast<int32_t*>(ws + l.roff);
  a.plan_order = reinterpret_cast<int32_t*>(ws + l.order);
  a.plan_pairs = reinterpret_cast<int32_t*>(ws + l.pairs);
  a.plan_cap = l.cap;
  return hip_status(launch_mapped_av_indexed(a, static_cast<hipStream_t>(stream)), "mapped_av_indexed launch");
}

int cma_onehot_mix(const int32_t* argmax, int32_t n_batch, int32_t n_recv, int32_t n_send, float* M,
                   void* stream) {
  if (n_batch < 0 || n_recv < 0 || n_send < 0) return fail(CMA_EINVAL, "negative size");
  if ((int64_t)n_batch * n_recv * n_send == 0) return CMA_OK;
  if (!argmax || !M) return fail(CMA_EINVAL, "NULL argmax or M");
  return hip_status(launch_onehot(argmax, n_batch, n_recv, n_send, M, static_cast<hipStream_t>(stream)),
                    "onehot_mix launch");
}

int cma_mapped_layers(int32_t n_layers, double ratio, int32_t* out, int32_t cap) {
  if (n_layers < 0 || !(ratio >= 0.0) || cap < 0 || (cap > 0 && !out))
    return fail(CMA_EINVAL, "bad arguments");
  auto half_up = [](double x) { return (int32_t)std::floor(x + 0.5); };
  const int32_t hi = half_up(0.8 * n_layers), lo = half_up(0.2 * n_layers);
  const int32_t avail = (n_layers - hi) + std::max(0, hi - lo);
  const int32_t want = std::min(half_up(ratio * n_layers), avail);
  int32_t k = 0;
  for (int32_t l = n_layers - 1; l >= hi && k < want; --l, ++k)
    if (k < cap) out[k] = l;
  for (int32_t l = lo; l < hi && k < want; ++l, ++k)
    if (k < cap) out[k] = l;
  return want;
}

int cma_mapping_plan(int32_t n, const int32_t* prompt_len, int32_t tau_e, int32_t tau_t,
                     int32_t* gen_before, int32_t* sim_len) {
  if (n < 0 || (n > 0 && (!prompt_len || !gen_before || !sim_len)) || tau_e < 0 || tau_t < 1)
    return fail(CMA_EINVAL, "bad arguments");
  for (int32_t i = 0; i < n; ++i)
    if (prompt_len[i] < 0) return fail(CMA_EINVAL, "negative prompt length at %d", i);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t gen = std::max(0, tau_e - prompt_len[i]);
    gen_before[i] = gen;
    sim_len[i] = std::min(prompt_len[i] + gen, tau_t);
  }
  return CMA_OK;
}

}  // extern "C"
