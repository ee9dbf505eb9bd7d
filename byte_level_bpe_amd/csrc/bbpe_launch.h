// Host-side kernel launcher shared by the encode and decode entry points.
#pragma once

#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>
#include <vector>

#include "../../include/bbpe.h"
#include "bbpe_tokenizer.h"

namespace bbpe {

#define HIP_OK(x)                               \
  do {                                          \
    if ((x) != hipSuccess) return BBPE_E_HIP;   \
  } while (0)

// Launches kernels on the caller's stream `st` (or, after use(), another);
// with timing enabled on the handle, every launch is bracketed by two events
// from the handle's pool.
struct Launcher {
  bbpe_tokenizer *t;
  hipStream_t st;
  hipStream_t cur = st;
  bool allow_timing = true;  // false: never record events, even with timing on
  std::vector<std::pair<int, size_t>> recs;  // (kernel index, first event)
  size_t next = 0;

  int kernel_index(const char *name) {
    for (size_t i = 0; i < t->t_names.size(); ++i)
      if (t->t_names[i] == name) return int(i);
    t->t_names.emplace_back(name);
    t->t_ms.push_back(0.0);
    t->t_launches.push_back(0);
    return int(t->t_names.size() - 1);
  }
  hipEvent_t event(size_t i) {
    while (t->t_events.size() <= i) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) e = nullptr;
      t->t_events.push_back(e);
    }
    return static_cast<hipEvent_t>(t->t_events[i]);
  }
  template <typename K, typename... A>
  void operator()(const char *name, K kernel, dim3 grid, dim3 block, A... args) {
    const bool timed = t->timing && allow_timing;
    if (timed) (void)hipEventRecord(event(next), cur);
    hipLaunchKernelGGL(kernel, grid, block, 0, cur, args...);
    if (timed) {
      (void)hipEventRecord(event(next + 1), cur);
      recs.emplace_back(kernel_index(name), next);
      next += 2;
    }
  }
  void use(hipStream_t s) { cur = s; }
  // The second stream (the handle's) and the caller's, and the fork/join
  // events between them (event 0: fork, 1: join).
  void use_aux() { cur = static_cast<hipStream_t>(t->aux_stream); }
  void use_main() { cur = st; }
  int record(int e) {
    HIP_OK(hipEventRecord(static_cast<hipEvent_t>(e == 0 ? t->ev_fork : t->ev_join), cur));
    return BBPE_OK;
  }
  int wait(int e) {
    HIP_OK(hipStreamWaitEvent(cur, static_cast<hipEvent_t>(e == 0 ? t->ev_fork : t->ev_join), 0));
    return BBPE_OK;
  }
  // after the streams have been synchronised
  void collect() {
    for (auto &r : recs) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, event(r.second), event(r.second + 1)) == hipSuccess) {
        t->t_ms[size_t(r.first)] += ms;
        t->t_launches[size_t(r.first)] += 1;
      }
    }
    recs.clear();
  }
};

// Builds a HIP graph of a kernel sequence instead of launching it: the same
// interface as Launcher, with its two streams as two chains of dependencies
// and its events as edges between them.  (No stream capture is involved, so
// other host threads' HIP work cannot interfere with the construction.)
struct GraphBuilder {
  hipGraph_t g = nullptr;
  hipGraphNode_t last[2] = {nullptr, nullptr};
  std::vector<hipGraphNode_t> pending[2];
  hipGraphNode_t ev[2] = {nullptr, nullptr};
  int cur = 0;
  int err = BBPE_OK;

  template <typename K, typename... A>
  void operator()(const char *, K kernel, dim3 grid, dim3 block, A... args) {
    if (err) return;
    std::tuple<A...> vals(args...);
    void *ptrs[sizeof...(A)];
    fill(ptrs, vals, std::index_sequence_for<A...>{});
    hipKernelNodeParams p{};
    p.func = reinterpret_cast<void *>(kernel);
    p.gridDim = grid;
    p.blockDim = block;
    p.sharedMemBytes = 0;
    p.kernelParams = ptrs;
    p.extra = nullptr;
    std::vector<hipGraphNode_t> deps = pending[cur];
    if (last[cur]) deps.push_back(last[cur]);
    hipGraphNode_t node = nullptr;
    if (hipGraphAddKernelNode(&node, g, deps.empty() ? nullptr : deps.data(), deps.size(), &p) !=
        hipSuccess) {
      err = BBPE_E_HIP;
      return;
    }
    last[cur] = node;
    pending[cur].clear();
  }
  template <typename Tu, size_t... I>
  static void fill(void **ptrs, Tu &vals, std::index_sequence<I...>) {
    ((ptrs[I] = static_cast<void *>(&std::get<I>(vals))), ...);
  }
  void use_aux() { cur = 1; }
  void use_main() { cur = 0; }
  int record(int e) {
    ev[e] = last[cur];
    return BBPE_OK;
  }
  int wait(int e) {
    if (ev[e]) pending[cur].push_back(ev[e]);
    return BBPE_OK;
  }
};

}  // namespace bbpe
