// Host-side kernel launcher shared by the encode and decode entry points.
#pragma once

#include <hip/hip_runtime.h>

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

}  // namespace bbpe
