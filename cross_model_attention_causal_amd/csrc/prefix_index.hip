// Prefix-hash index of compressed sender states (MapFlow, storage and execution:
// the second component). The block-sparse rows a sender leaves differ in number
// per layer and position; the index keys each cached block-row by a hash that
// carries the whole preceding context, so a receiver (or a later request with
// the same prefix) finds the rows it can reuse, and one sender state can serve
// several downstream models.
//
// Host code only. Keys: (layer, chained hash of the 64-token blocks up to and
// including the block-row's own block). The chained hash is 64-bit FNV-1a (the
// Fowler-Noll-Vo hash, variant 1a) over the previous block's hash (8 bytes,
// little-endian; the caller's seed for block 0) followed by the block's 64
// token ids (4 bytes each, little-endian). Values: for each sender head, the
// first stored block of the row in the caller's block pool and the row's block
// count (what row_ptr / row_end of a block-sparse source take). Entries live
// until erased or evicted; lookups refresh an entry's recency, and the caller
// evicts least-recently-used entries explicitly (it owns the pool space they
// name). Thread-safe: every call takes the index's lock.
#include <cstdint>
#include <cstring>
#include <list>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "cma.h"

namespace {

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

uint64_t fnv1a_bytes(uint64_t h, const unsigned char* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

uint64_t fnv1a_u64(uint64_t h, uint64_t x) {
  unsigned char b[8];
  for (int i = 0; i < 8; ++i) b[i] = (unsigned char)(x >> (8 * i));
  return fnv1a_bytes(h, b, 8);
}

uint64_t fnv1a_i32(uint64_t h, int32_t x) {
  const uint32_t u = (uint32_t)x;
  unsigned char b[4];
  for (int i = 0; i < 4; ++i) b[i] = (unsigned char)(u >> (8 * i));
  return fnv1a_bytes(h, b, 4);
}

struct Key {
  int32_t layer;
  uint64_t hash;
  bool operator==(const Key& o) const { return layer == o.layer && hash == o.hash; }
};
struct KeyHash {
  size_t operator()(const Key& k) const { return (size_t)(k.hash ^ (0x9e3779b97f4a7c15ull * (uint32_t)k.layer)); }
};

}  // namespace

struct cma_prefix_index {
  int32_t n_heads;
  int64_t capacity;
  std::mutex mu;
  struct Entry {
    Key key;
    std::vector<int32_t> begin, count;
  };
  std::list<Entry> lru;  // most recently used first
  std::unordered_map<Key, std::list<Entry>::iterator, KeyHash> map;
};

extern "C" {

int cma_prefix_hashes(const int32_t* tokens, int64_t n_tokens, uint64_t seed, uint64_t* hashes) {
  if (n_tokens < 0 || (n_tokens >= 64 && (!tokens || !hashes))) return CMA_EINVAL;
  uint64_t prev = seed;
  for (int64_t b = 0; b < n_tokens / 64; ++b) {
    uint64_t h = fnv1a_u64(kFnvOffset, prev);
    for (int t = 0; t < 64; ++t) h = fnv1a_i32(h, tokens[64 * b + t]);
    hashes[b] = h;
    prev = h;
  }
  return CMA_OK;
}

uint64_t cma_fnv1a64(const void* data, size_t n_bytes) {
  return fnv1a_bytes(kFnvOffset, static_cast<const unsigned char*>(data), data ? n_bytes : 0);
}

cma_prefix_index* cma_prefix_index_create(int32_t n_heads, int64_t capacity) {
  if (n_heads < 1 || capacity < 1) return nullptr;
  cma_prefix_index* ix = new (std::nothrow) cma_prefix_index();
  if (!ix) return nullptr;
  ix->n_heads = n_heads;
  ix->capacity = capacity;
  return ix;
}

void cma_prefix_index_destroy(cma_prefix_index* ix) { delete ix; }

int64_t cma_prefix_index_size(cma_prefix_index* ix) {
  if (!ix) return CMA_EINVAL;
  std::lock_guard<std::mutex> lk(ix->mu);
  return (int64_t)ix->map.size();
}

int cma_prefix_index_insert(cma_prefix_index* ix, int32_t layer, uint64_t hash, const int32_t* begin,
                            const int32_t* count) {
  if (!ix || !begin || !count) return CMA_EINVAL;
  for (int32_t h = 0; h < ix->n_heads; ++h)
    if (begin[h] < 0 || count[h] < 0) return CMA_EINVAL;
  std::lock_guard<std::mutex> lk(ix->mu);
  const Key key{layer, hash};
  auto it = ix->map.find(key);
  if (it != ix->map.end()) {  // the same prefix again: the new location replaces the old
    it->second->begin.assign(begin, begin + ix->n_heads);
    it->second->count.assign(count, count + ix->n_heads);
    ix->lru.splice(ix->lru.begin(), ix->lru, it->second);
    return CMA_OK;
  }
  if ((int64_t)ix->map.size() >= ix->capacity) return CMA_ENOSPC;
  ix->lru.push_front({key, std::vector<int32_t>(begin, begin + ix->n_heads),
                      std::vector<int32_t>(count, count + ix->n_heads)});
  ix->map.emplace(key, ix->lru.begin());
  return CMA_OK;
}

int64_t cma_prefix_index_lookup(cma_prefix_index* ix, int32_t layer, const uint64_t* hashes, int64_t n,
                                int32_t* begin, int32_t* count) {
  if (!ix || n < 0 || (n > 0 && !hashes)) return CMA_EINVAL;
  std::lock_guard<std::mutex> lk(ix->mu);
  int64_t hits = 0;
  for (; hits < n; ++hits) {
    auto it = ix->map.find(Key{layer, hashes[hits]});
    if (it == ix->map.end()) break;
    ix->lru.splice(ix->lru.begin(), ix->lru, it->second);
    if (begin) std::memcpy(begin + hits * ix->n_heads, it->second->begin.data(), ix->n_heads * sizeof(int32_t));
    if (count) std::memcpy(count + hits * ix->n_heads, it->second->count.data(), ix->n_heads * sizeof(int32_t));
  }
  return hits;
}

int cma_prefix_index_erase(cma_prefix_index* ix, int32_t layer, uint64_t hash) {
  if (!ix) return CMA_EINVAL;
  std::lock_guard<std::mutex> lk(ix->mu);
  auto it = ix->map.find(Key{layer, hash});
  if (it == ix->map.end()) return 0;
  ix->lru.erase(it->second);
  ix->map.erase(it);
  return 1;
}

int cma_prefix_index_evict_lru(cma_prefix_index* ix, int32_t* layer, uint64_t* hash, int32_t* begin,
                               int32_t* count) {
  if (!ix) return CMA_EINVAL;
  std::lock_guard<std::mutex> lk(ix->mu);
  if (ix->lru.empty()) return 0;
  auto& e = ix->lru.back();
  if (layer) *layer = e.key.layer;
  if (hash) *hash = e.key.hash;
  if (begin) std::memcpy(begin, e.begin.data(), ix->n_heads * sizeof(int32_t));
  if (count) std::memcpy(count, e.count.data(), ix->n_heads * sizeof(int32_t));
  ix->map.erase(e.key);
  ix->lru.pop_back();
  return 1;
}

}  // extern "C"
