// Host driver for the prefix-hash index, built with the host sanitizers
// (AddressSanitizer + UndefinedBehaviorSanitizer, or ThreadSanitizer) together
// with the library's prefix_index source. It runs a script of operations read
// from a file and prints one result line per operation (the test replays the
// same script on the oracle's model of the index and compares the lines), then
// calls the API with invalid arguments and hammers one index from several
// threads (no results compared: the sanitizers watch memory and locking).
//
// Script lines (whitespace-separated integers; hashes in decimal):
//   C n_heads capacity              create the index (replacing the previous one)
//   H seed n tok_0 .. tok_{n-1}     prefix hashes      -> "H h_0 .. h_{b-1}"
//   I layer hash b_0 c_0 .. b_k c_k insert             -> "I status"
//   L layer n hash_0 .. hash_{n-1}  lookup             -> "L hits b c .. (per hit, per head)"
//   E layer hash                    erase              -> "E result"
//   V                               evict LRU          -> "V 0" or "V 1 layer hash b c .."
//   S                               size               -> "S n"
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <thread>
#include <vector>

#include "cma.h"

namespace {

int fail(const char* what) {
  std::fprintf(stderr, "driver: %s\n", what);
  return 2;
}

int run_script(FILE* in) {
  cma_prefix_index* ix = nullptr;
  int32_t n_heads = 0;
  char op[4];
  while (std::fscanf(in, "%3s", op) == 1) {
    if (op[0] == 'C') {
      long long cap = 0;
      if (std::fscanf(in, "%d %lld", &n_heads, &cap) != 2) return fail("bad C");
      if (ix) cma_prefix_index_destroy(ix);
      ix = cma_prefix_index_create(n_heads, cap);
      if (!ix) return fail("create failed");
    } else if (op[0] == 'H') {
      unsigned long long seed = 0;
      long long n = 0;
      if (std::fscanf(in, "%llu %lld", &seed, &n) != 2 || n < 0) return fail("bad H");
      std::vector<int32_t> tok((size_t)n);
      for (auto& t : tok)
        if (std::fscanf(in, "%d", &t) != 1) return fail("bad H token");
      std::vector<uint64_t> h((size_t)(n / 64));
      const int st = cma_prefix_hashes(tok.data(), n, seed, h.data());
      std::printf("H");
      if (st < 0) std::printf(" status %d", st);
      for (uint64_t x : h) std::printf(" %" PRIu64, x);
      std::printf("\n");
    } else if (op[0] == 'I') {
      int32_t layer = 0;
      unsigned long long hash = 0;
      if (std::fscanf(in, "%d %llu", &layer, &hash) != 2) return fail("bad I");
      std::vector<int32_t> b((size_t)n_heads), c((size_t)n_heads);
      for (int32_t k = 0; k < n_heads; ++k)
        if (std::fscanf(in, "%d %d", &b[(size_t)k], &c[(size_t)k]) != 2) return fail("bad I pair");
      std::printf("I %d\n", cma_prefix_index_insert(ix, layer, hash, b.data(), c.data()));
    } else if (op[0] == 'L') {
      int32_t layer = 0;
      long long n = 0;
      if (std::fscanf(in, "%d %lld", &layer, &n) != 2 || n < 0) return fail("bad L");
      std::vector<uint64_t> h((size_t)n);
      for (auto& x : h) {
        unsigned long long v = 0;
        if (std::fscanf(in, "%llu", &v) != 1) return fail("bad L hash");
        x = v;
      }
      std::vector<int32_t> b((size_t)(n * n_heads)), c((size_t)(n * n_heads));
      const int64_t hits = cma_prefix_index_lookup(ix, layer, h.data(), n, b.data(), c.data());
      std::printf("L %" PRId64, hits);
      for (int64_t i = 0; i < hits * n_heads; ++i) std::printf(" %d %d", b[(size_t)i], c[(size_t)i]);
      std::printf("\n");
    } else if (op[0] == 'E') {
      int32_t layer = 0;
      unsigned long long hash = 0;
      if (std::fscanf(in, "%d %llu", &layer, &hash) != 2) return fail("bad E");
      std::printf("E %d\n", cma_prefix_index_erase(ix, layer, hash));
    } else if (op[0] == 'V') {
      int32_t layer = -1;
      uint64_t hash = 0;
      std::vector<int32_t> b((size_t)n_heads), c((size_t)n_heads);
      const int r = cma_prefix_index_evict_lru(ix, &layer, &hash, b.data(), c.data());
      std::printf("V %d", r);
      if (r == 1) {
        std::printf(" %d %" PRIu64, layer, hash);
        for (int32_t k = 0; k < n_heads; ++k) std::printf(" %d %d", b[(size_t)k], c[(size_t)k]);
      }
      std::printf("\n");
    } else if (op[0] == 'S') {
      std::printf("S %" PRId64 "\n", cma_prefix_index_size(ix));
    } else {
      return fail("unknown op");
    }
  }
  if (ix) cma_prefix_index_destroy(ix);
  return 0;
}

// Invalid arguments: every call must refuse them with a negative status (or
// NULL / 0) and touch no memory it was not given.
int check_invalid() {
  uint64_t h[2] = {1, 2};
  int32_t b[2] = {0, 0}, c[2] = {1, 1};
  if (cma_prefix_index_create(0, 4) || cma_prefix_index_create(2, -1)) return fail("create accepted bad args");
  if (cma_prefix_hashes(nullptr, 64, 0, h) >= 0) return fail("hashes accepted NULL tokens");
  if (cma_prefix_hashes(b, -1, 0, h) >= 0) return fail("hashes accepted n < 0");
  if (cma_prefix_index_insert(nullptr, 0, 1, b, c) >= 0) return fail("insert accepted NULL index");
  if (cma_prefix_index_lookup(nullptr, 0, h, 2, b, c) >= 0) return fail("lookup accepted NULL index");
  if (cma_prefix_index_size(nullptr) >= 0) return fail("size accepted NULL index");
  cma_prefix_index* ix = cma_prefix_index_create(2, 2);
  if (!ix) return fail("create failed");
  const int32_t neg[2] = {-1, 0};
  if (cma_prefix_index_insert(ix, 0, 1, neg, c) >= 0) return fail("insert accepted a negative begin");
  if (cma_prefix_index_insert(ix, 0, 1, b, nullptr) >= 0) return fail("insert accepted NULL count");
  if (cma_prefix_index_lookup(ix, 0, h, -1, b, c) >= 0) return fail("lookup accepted n < 0");
  if (cma_prefix_index_lookup(ix, 0, nullptr, 2, b, c) >= 0) return fail("lookup accepted NULL hashes");
  if (cma_prefix_index_lookup(ix, 0, h, 2, nullptr, nullptr) != 0) return fail("lookup of an empty index");
  cma_prefix_index_destroy(ix);
  cma_prefix_index_destroy(nullptr);
  return 0;
}

// Several threads share one small index (so that inserts meet a full index and
// evictions race with lookups).
int hammer() {
  constexpr int kThreads = 8, kIters = 4000, kHeads = 3;
  cma_prefix_index* ix = cma_prefix_index_create(kHeads, 64);
  if (!ix) return fail("create failed");
  std::vector<std::thread> th;
  for (int t = 0; t < kThreads; ++t) {
    th.emplace_back([ix, t] {
      uint64_t x = 0x9e3779b97f4a7c15ull * (uint64_t)(t + 1);
      int32_t b[4 * kHeads], c[4 * kHeads];
      for (int i = 0; i < kIters; ++i) {
        x ^= x << 13;
        x ^= x >> 7;
        x ^= x << 17;
        const int32_t layer = (int32_t)(x % 3);
        const uint64_t key = (x >> 8) % 97;
        for (int k = 0; k < kHeads; ++k) {
          b[k] = (int32_t)(key * 10 + (uint64_t)k);
          c[k] = k + 1;
        }
        switch (x % 5) {
          case 0:
          case 1:
            if (cma_prefix_index_insert(ix, layer, key, b, c) == CMA_ENOSPC)
              cma_prefix_index_evict_lru(ix, nullptr, nullptr, nullptr, nullptr);
            break;
          case 2: {
            const uint64_t hs[4] = {key, key + 1, key + 2, key + 3};
            cma_prefix_index_lookup(ix, layer, hs, 4, b, c);
            break;
          }
          case 3:
            cma_prefix_index_erase(ix, layer, key);
            break;
          default:
            cma_prefix_index_size(ix);
        }
      }
    });
  }
  for (auto& t : th) t.join();
  const int64_t n = cma_prefix_index_size(ix);
  cma_prefix_index_destroy(ix);
  return (n >= 0 && n <= 64) ? 0 : fail("size out of range after the threads");
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) return fail("usage: driver SCRIPT");
  FILE* in = std::fopen(argv[1], "r");
  if (!in) return fail("cannot open the script");
  int rc = run_script(in);
  std::fclose(in);
  if (rc == 0) rc = check_invalid();
  if (rc == 0) rc = hammer();
  return rc;
}
