// Per-word set-up shared by the front-end kernels (gfx950): the lane's text
// window, the segment starts around it and its class masks.
//
// The first front-end kernel computes the two costly parts for every word it
// owns and stores them in the workspace: the multi-byte part of the masks
// (a per-character decode and two class-table loads) for words holding a
// byte >= 0x80, and the segment marks (two binary searches over the segment
// offsets) when there is more than one segment.  The later kernels read them
// back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bbpe_classify.h"
#include "bbpe_kernels.h"

namespace bbpe {

// FIRST: compute and store (owners only); else read back.  Words outside
// [0, n_words) (halo lanes at the ends of the text) always compute.
template <bool FIRST>
__device__ __forceinline__ void word_setup(const EncodeArgs &a, int64_t w, bool owned, Window &win,
                                           uint64_t &seg_lo, uint64_t &seg_hi, uint32_t &seg_at,
                                           WordMasks &m) {
  const int64_t base = w * 64;
  const bool in = w >= 0 && w < int64_t(a.n_words);
  load_window(a.text, a.n, base, win);
  // the first kernel stages the wave's bytes in LDS for the multi-byte
  // decoder (one wave per workgroup, lane = threadIdx.x at consecutive words)
  const SlowStage *st = nullptr;
  int64_t lo = 0;
  if (FIRST) {
    __shared__ SlowStage stage;
    stage_fill(stage, a.T, win, int(threadIdx.x));
    st = &stage;
    lo = base - int64_t(threadIdx.x) * 64 - 16;
  }
  if (a.n_seg > 1 && in && !FIRST) {
    const ulonglong2 v = reinterpret_cast<const ulonglong2 *>(a.ws.wseg)[w];
    seg_lo = v.x;
    seg_hi = v.y;
    seg_at = a.ws.wseg_at[w];
  } else {
    segment_marks(a.seg_off, a.n_seg, base, seg_lo, seg_hi, seg_at);
    if (FIRST && a.n_seg > 1 && owned) {
      reinterpret_cast<ulonglong2 *>(a.ws.wseg)[w] = ulonglong2{seg_lo, seg_hi};
      a.ws.wseg_at[w] = seg_at;
    }
  }
  // (a word outside [0, n_words) has no valid byte: classify_word returns
  // before the multi-byte part, so later kernels read a record only for
  // words that have one)
  uint64_t *rec = in ? a.ws.wslow + uint64_t(w) * SLOW_WORDS : nullptr;
  classify_word<FIRST>(a.T, a.text, win, base, a.n, seg_lo, seg_hi, m, FIRST ? nullptr : rec,
                       (FIRST && owned) ? rec : nullptr, st, lo);
}

}  // namespace bbpe
