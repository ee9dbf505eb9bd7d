// Test infrastructure: the CPU baseline's multi-core row.  Runs the plain
// oracle (oracle_encode, unchanged and single-threaded per call) over
// independent units of a workload -- segments, and the 400,000-character
// windows of a segment, which tiktoken-safe chunking encodes as texts of
// their own (Baseten page, "Why Kimi K3 tokenization is non-trivial"; each
// such chunk on its own core: "Where the speed comes from") -- on K
// std::threads, one oracle handle per thread, units taken in order from a
// shared counter.  The ids of the units are concatenated in unit order.
#include <stdint.h>

#include <atomic>
#include <chrono>
#include <thread>
#include <vector>

extern "C" int oracle_encode(void *h, const uint8_t *text, const uint64_t *seg_off,
                             const uint8_t *allow, uint32_t nseg, int safe, int32_t *ids,
                             uint64_t cap, int64_t *id_off, uint64_t *n_ids, uint64_t *err_seg,
                             uint64_t *err_byte);

extern "C" {

// handles[k]: one oracle per thread (k < n_threads); unit u is
// text[unit_off[u] .. unit_off[u+1]) with allow[u].  Writes the
// concatenated ids (capacity cap) and their count; *seconds is the wall
// time of the threaded section (threads started to threads joined).
// Returns 0, or the first unit's nonzero oracle status.
int oracle_encode_units_mt(void **handles, int n_threads, const uint8_t *text,
                           const uint64_t *unit_off, const uint8_t *allow, uint32_t n_units,
                           int safe, int32_t *ids, uint64_t cap, uint64_t *n_ids,
                           double *seconds) {
  if (n_threads < 1) return -1;
  std::vector<std::vector<int32_t>> out(n_units);
  std::vector<int> status(n_units, 0);
  std::atomic<uint32_t> next{0};
  auto worker = [&](int k) {
    for (;;) {
      const uint32_t u = next.fetch_add(1);
      if (u >= n_units) return;
      const uint64_t len = unit_off[u + 1] - unit_off[u];
      const uint64_t off[2] = {0, len};
      std::vector<int32_t> &v = out[u];
      v.resize(len);  // a unit of len bytes yields at most len ids
      uint64_t n = 0, es = 0, eb = 0;
      status[u] = oracle_encode(handles[k], text + unit_off[u], off, allow + u, 1, safe,
                                v.data(), len, nullptr, &n, &es, &eb);
      v.resize(status[u] ? 0 : n);
    }
  };
  const auto t0 = std::chrono::steady_clock::now();
  std::vector<std::thread> th;
  for (int k = 0; k < n_threads; ++k) th.emplace_back(worker, k);
  for (auto &t : th) t.join();
  const auto t1 = std::chrono::steady_clock::now();
  *seconds = std::chrono::duration<double>(t1 - t0).count();
  uint64_t total = 0;
  for (uint32_t u = 0; u < n_units; ++u) {
    if (status[u]) return status[u];
    total += out[u].size();
  }
  *n_ids = total;
  if (total > cap) return -5;
  uint64_t p = 0;
  for (uint32_t u = 0; u < n_units; ++u)
    for (int32_t x : out[u]) ids[p++] = x;
  return 0;
}

}  // extern "C"
