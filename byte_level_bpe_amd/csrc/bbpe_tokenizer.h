// Host-side tokenizer handle (opaque to callers of bbpe.h).
#pragma once

#include <stdint.h>

#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "bbpe_internal.h"

struct bbpe_tokenizer {
  int grammar = 0;
  uint32_t n_ranks = 0;
  int32_t max_id = -1;
  // decode map: id -> (offset into dec_blob, length); dense when ids are dense
  std::vector<uint8_t> dec_blob;
  std::vector<uint64_t> dec_dense;  // (off << 8) | len, or ~0 when absent
  std::unordered_map<int32_t, uint64_t> dec_sparse;
  bool dense = true;
  // specials
  std::vector<std::string> sp;
  std::vector<int32_t> sp_id;
  // device image, built on the host at load time and copied by upload
  bbpe::ImageLayout layout{};
  std::vector<uint8_t> image;
  const uint8_t *d_image = nullptr;
  bbpe::DevTables dev{};
  uint32_t max_key_len = 0;
  uint32_t dev_dec_n = 0;  // largest rank + 1 (the device decode table's size)
  uint32_t n_self_consistent = 0;
  // per-kernel timing (diagnostics)
  bool timing = false;
  std::vector<std::string> t_names;
  std::vector<double> t_ms;
  std::vector<uint64_t> t_launches;
  std::vector<void *> t_events;  // hipEvent_t pool, two per launch
  // second stream for merge tiers that run beside the short tier, and the
  // two events that fork it from and join it back to the caller's stream
  // (created at the first encode, on the device current then)
  void *aux_stream = nullptr;
  void *ev_fork = nullptr, *ev_join = nullptr;
  // The status block of the last call, written by its last kernel into
  // pinned host memory (allocated by bbpe_upload_tables): read after the
  // call's one stream synchronisation.  host_status_dev is its device
  // address.
  void *host_status = nullptr, *host_status_dev = nullptr;
  // The last encode's kernel sequence (both streams) as an instantiated HIP
  // graph, and the arguments it was built with: a call with the same
  // arguments replays it with one launch.
  void *graph_exec = nullptr;
  std::vector<uint8_t> graph_key;
  bool graph_broken = false;  // building one failed: launch kernels directly
  // The word cache kept across calls (BBPE_KEEP_WORD_CACHE): allocated on the
  // device current at the first call that asks for it, freed by bbpe_free.
  void *wcache = nullptr;
  uint64_t wc_last_hits = 0;  // units the last such call settled from it
  // Encodes enqueued by bbpe_encode_segments_async and not yet waited for,
  // the stream they are on (every call of the handle uses it until the
  // wait), and whether the last of them kept the word cache.
  uint32_t inflight = 0;
  void *async_stream = nullptr;
  bool async_keep = false;
  // Every entry point that enqueues work or touches the mutable state above
  // (second stream, fork/join events, timing records) holds this lock for
  // the whole call, so that host threads sharing a handle never interleave
  // their fork/join events or timing records; such calls run one after the
  // other.
  std::mutex mu;
};

namespace bbpe {
// The calling thread's last BBPE_E_UTF8 on a handle (bbpe_error_detail).
void set_last_utf8_error(const bbpe_tokenizer *t, uint32_t seg, uint64_t byte);
// Hash of a host key (same function the kernels apply to text slices).
uint64_t hash_key(const uint8_t *p, uint32_t len);
}  // namespace bbpe
