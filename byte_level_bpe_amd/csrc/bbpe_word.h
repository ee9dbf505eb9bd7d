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

// Segment starts at window indices -8..119 of every lane of the wave, and
// the segment holding each lane's first byte (what segment_marks gives one
// lane), found by the wave together: a 64-ary search for the first segment
// start at or after lane 0's window, then the starts up to the end of lane
// 63's window, read 64 at a time and sorted to lanes through LDS.  Every
// lane calls this (lane = threadIdx.x at consecutive words).  Offsets out of
// order give some bounded result (seg_at < n_seg); the call is then refused.
__device__ __forceinline__ void wave_segment_marks(const uint64_t *__restrict__ seg_off, uint32_t n_seg,
                                                   int64_t base, int lane, SlowStage &st,
                                                   uint64_t &lo, uint64_t &hi, uint32_t &seg_at) {
  const int64_t from0 = base - 64 * int64_t(lane) - 8;  // lane 0's window start
  const int64_t end = from0 + 63 * 64 + 128;           // lane 63's window end
  st.sq.sm[0][lane] = 0;
  st.sq.sm[1][lane] = 0;
  st.sq.sh[lane] = 0;
  // first s in [0, n_seg) with seg_off[s] >= from0
  uint32_t a = 0, b = n_seg;
  while (b - a > 64) {
    const uint32_t step = (b - a + 63) / 64;
    const uint64_t idx = uint64_t(a) + uint64_t(lane) * step;
    const bool p = idx < b && int64_t(seg_off[idx]) < from0;
    const uint32_t c = uint32_t(__popcll(__ballot(p)));
    const uint32_t a0 = a;
    if (c == 0) {
      b = a;
    } else {
      a = a0 + (c - 1) * step + 1;
      b = uint32_t(min(uint64_t(b), uint64_t(a0) + uint64_t(c) * step));
    }
  }
  {
    const uint32_t idx = a + uint32_t(lane);
    const bool p = idx < b && int64_t(seg_off[idx]) < from0;
    a += uint32_t(__popcll(__ballot(p)));
  }
  __syncthreads();
  // starts from s = a on: lane l1 = d / 64 sees one in the low word of its
  // window and lane l1 - 1 in the high word (d = offset - from0); it counts
  // toward seg_at of the lanes whose first byte is at or after it
  for (uint64_t j0 = a; j0 < n_seg; j0 += 64) {
    const uint64_t idx = j0 + uint64_t(lane);
    const int64_t o = idx < n_seg ? int64_t(seg_off[idx]) : end;
    const bool in = o < end;
    if (in && o >= from0) {
      const int64_t d = o - from0;
      const int l1 = int(d >> 6);
      const uint64_t m = bit(int(d & 63));
      if (l1 < 64) atomicOr(reinterpret_cast<unsigned long long *>(&st.sq.sm[0][l1]), m);
      if (l1 >= 1) atomicOr(reinterpret_cast<unsigned long long *>(&st.sq.sm[1][l1 - 1]), m);
      const int64_t lf = d <= 8 ? 0 : (d - 8 + 63) >> 6;
      if (lf < 64) atomicAdd(&st.sq.sh[lf], 1u);
    } else if (in) {
      atomicAdd(&st.sq.sh[0], 1u);
    }
    if (!((__ballot(in) >> 63) & 1)) break;
  }
  __syncthreads();
  lo = st.sq.sm[0][lane];
  hi = st.sq.sm[1][lane];
  const uint32_t cum = a + wave_incl_sum(st.sq.sh[lane], lane);
  seg_at = cum > 0 ? cum - 1 : 0;
}

// The window `win` is loaded by the caller (load_window at w * 64), as early
// as it can be.  FIRST: compute and store (owners only); else read back.  Words outside
// [0, n_words) (halo lanes at the ends of the text) always compute.
template <bool FIRST>
__device__ __forceinline__ void word_setup(const EncodeArgs &a, int64_t w, bool owned, Window &win,
                                           uint64_t &seg_lo, uint64_t &seg_hi, uint32_t &seg_at,
                                           WordMasks &m) {
  const int64_t base = w * 64;
  const bool in = w >= 0 && w < int64_t(a.n_words);
  // the first kernel's wave works together (one wave per workgroup, lane =
  // threadIdx.x at consecutive words) in LDS: the segment-start search and
  // the multi-byte decoder
  SlowStage *st = nullptr;
  if (FIRST) {
    __shared__ SlowStage stage;
    st = &stage;
    wave_segment_marks(a.seg_off, a.n_seg, base, int(threadIdx.x), *st, seg_lo, seg_hi, seg_at);
    if (a.n_seg > 1 && owned) {
      reinterpret_cast<ulonglong2 *>(a.ws.wseg)[w] = ulonglong2{seg_lo, seg_hi};
      a.ws.wseg_at[w] = seg_at;
    }
  } else if (a.n_seg > 1 && in) {
    const ulonglong2 v = reinterpret_cast<const ulonglong2 *>(a.ws.wseg)[w];
    seg_lo = v.x;
    seg_hi = v.y;
    seg_at = a.ws.wseg_at[w];
  } else {
    segment_marks(a.seg_off, a.n_seg, base, seg_lo, seg_hi, seg_at);
  }
  // (a word outside [0, n_words) has no valid byte: classify_word returns
  // before the multi-byte part, so later kernels read a record only for
  // words that have one)
  uint64_t *rec = in ? a.ws.wslow + uint64_t(w) * SLOW_WORDS : nullptr;
  classify_word<FIRST>(a.T, a.text, win, base, a.n, seg_lo, seg_hi, m, FIRST ? nullptr : rec,
                       (FIRST && owned) ? rec : nullptr, st);
}

}  // namespace bbpe
