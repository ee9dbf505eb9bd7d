// Device helpers for the gfx950 kernels: the per-lane 64-byte text window,
// UTF-8 decoding into per-word class bitmasks, and wave64 scans.
//
// Layout: one lane owns one "word" of 64 consecutive text bytes; bit i of a
// 64-bit mask describes byte (64*word + i).  A character's class bits are set
// on all of its bytes; LEAD marks its first byte.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bbpe_internal.h"

namespace bbpe {

// ---------------------------------------------------------------------------
// Cross-word shifts.  shl(x, prev, k): bit i takes x's bit i-k (bytes before,
// from the previous word for i < k).  shr(x, next, k): bit i takes bit i+k.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t shl(uint64_t x, uint64_t prev, int k) {
  return (x << k) | (prev >> (64 - k));
}
__device__ __forceinline__ uint64_t shr(uint64_t x, uint64_t next, int k) {
  return (x >> k) | (next << (64 - k));
}
__device__ __forceinline__ uint64_t bit(int i) { return uint64_t(1) << i; }

__device__ __forceinline__ uint64_t shfl_up64(uint64_t v, int d) {
  return __shfl_up(static_cast<unsigned long long>(v), d, 64);
}
__device__ __forceinline__ uint64_t shfl_down64(uint64_t v, int d) {
  return __shfl_down(static_cast<unsigned long long>(v), d, 64);
}

// Inclusive scans over the 64 lanes of the wave (every lane active) by DPP
// moves: row shifts by 1, 2, 4 and 8 within each row of 16 lanes, then the
// last lane of rows 0 and 2 into rows 1 and 3, then lane 31 into rows 2 and
// 3.  A lane without a source in a step takes the identity.  op(earlier,
// later).  (Shuffles through the LDS crossbar wait for it at every step.)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v, uint32_t id) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(id), int(v), CTRL, ROW_MASK, 0xf, false));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_mov(uint64_t v, uint64_t id) {
  return uint64_t(dpp_mov<CTRL, ROW_MASK>(uint32_t(v), uint32_t(id))) |
         (uint64_t(dpp_mov<CTRL, ROW_MASK>(uint32_t(v >> 32), uint32_t(id >> 32))) << 32);
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_incl_scan(T v, T id, Op op) {
  v = op(dpp_mov<0x111, 0xf>(v, id), v);  // row_shr:1
  v = op(dpp_mov<0x112, 0xf>(v, id), v);  // row_shr:2
  v = op(dpp_mov<0x114, 0xf>(v, id), v);  // row_shr:4
  v = op(dpp_mov<0x118, 0xf>(v, id), v);  // row_shr:8
  v = op(dpp_mov<0x142, 0xa>(v, id), v);  // row_bcast:15
  v = op(dpp_mov<0x143, 0xc>(v, id), v);  // row_bcast:31
  return v;
}

// Inclusive prefix sum over the 64 lanes of the wave.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v, int lane) {
  (void)lane;
  return wave_incl_scan(v, 0u, [](uint32_t x, uint32_t y) { return x + y; });
}
// lane 63's value, in every lane
__device__ __forceinline__ uint32_t lane63(uint32_t v) { return uint32_t(__builtin_amdgcn_readlane(int(v), 63)); }
__device__ __forceinline__ uint64_t lane63(uint64_t v) {
  return uint64_t(lane63(uint32_t(v))) | (uint64_t(lane63(uint32_t(v >> 32))) << 32);
}
// op over the 64 lanes, in every lane (every lane active)
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, T id, Op op) {
  return lane63(wave_incl_scan(v, id, op));
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return wave_reduce(v, 0u, [](uint32_t x, uint32_t y) { return x + y; });
}
// Inclusive scan of op (associative, identity id) over the threads of a
// block of NT threads in thread order: a wave scan by shuffles, then the
// first wave scans the wave totals (sh: 2 * NT/64 + 1 entries of LDS).
// total: op over all threads.
template <uint32_t NT, typename T, typename Op>
__device__ __forceinline__ T block_incl_scan(T v, T id, Op op, T *sh, T &total) {
  constexpr uint32_t NW = NT / 64;
  const int lane = int(threadIdx.x & 63);
  const uint32_t wv = threadIdx.x / 64;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const T o = __shfl_up(v, d, 64);
    if (lane >= d) v = op(o, v);
  }
  if (lane == 63) sh[wv] = v;
  __syncthreads();
  if (wv == 0) {
    T x = uint32_t(lane) < NW ? sh[lane] : id;
#pragma unroll
    for (int d = 1; d < int(NW); d <<= 1) {
      const T o = __shfl_up(x, d, 64);
      if (lane >= d) x = op(o, x);
    }
    T ex = __shfl_up(x, 1, 64);
    if (lane == 0) ex = id;
    if (uint32_t(lane) < NW) sh[NW + lane] = ex;
    if (uint32_t(lane) == NW - 1) sh[2 * NW] = x;
  }
  __syncthreads();
  const T pre = sh[NW + wv];
  total = sh[2 * NW];
  __syncthreads();
  return op(pre, v);
}
// The same in reverse thread order (thread NT-1 first): op(later, earlier).
template <uint32_t NT, typename T, typename Op>
__device__ __forceinline__ T block_incl_scan_rev(T v, T id, Op op, T *sh) {
  constexpr uint32_t NW = NT / 64;
  const int lane = int(threadIdx.x & 63);
  const uint32_t wv = threadIdx.x / 64;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const T o = __shfl_down(v, d, 64);
    if (lane + d < 64) v = op(o, v);
  }
  if (lane == 0) sh[wv] = v;
  __syncthreads();
  if (wv == 0) {
    T x = uint32_t(lane) < NW ? sh[lane] : id;
#pragma unroll
    for (int d = 1; d < int(NW); d <<= 1) {
      const T o = __shfl_down(x, d, 64);
      if (uint32_t(lane + d) < NW) x = op(o, x);
    }
    T ex = __shfl_down(x, 1, 64);
    if (uint32_t(lane) + 1 >= NW) ex = id;
    if (uint32_t(lane) < NW) sh[NW + lane] = ex;
  }
  __syncthreads();
  const T pre = sh[NW + wv];
  __syncthreads();
  return op(pre, v);
}

__device__ __forceinline__ int64_t wave_incl_max(int64_t v, int lane) {
  (void)lane;
  const uint64_t lo = uint64_t(INT64_MIN);  // the identity of max
  return int64_t(wave_incl_scan(uint64_t(v), lo, [](uint64_t x, uint64_t y) {
    return int64_t(x) > int64_t(y) ? x : y;
  }));
}

// ---------------------------------------------------------------------------
// 96-byte text window of a lane: bytes [base-16, base+80) of the text, zero
// outside [0, n).  Loaded with 16-byte vector loads where fully in range.
// ---------------------------------------------------------------------------
struct Window {
  uint32_t w[24];
  __device__ __forceinline__ uint32_t at(int k) const {  // k in [-16, 80)
    const int q = k + 16;
    return (w[q >> 2] >> ((q & 3) * 8)) & 0xFFu;
  }
};

__device__ __forceinline__ void load_window(const uint8_t *__restrict__ text, uint64_t n,
                                            int64_t base, Window &win) {
  if (base >= 16 && uint64_t(base) + 80 <= n) {
    const uint4 *p = reinterpret_cast<const uint4 *>(text + base - 16);
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      const uint4 v = p[q];
      win.w[4 * q + 0] = v.x;
      win.w[4 * q + 1] = v.y;
      win.w[4 * q + 2] = v.z;
      win.w[4 * q + 3] = v.w;
    }
  } else {
    // Near the ends of the text: every dword load is issued unconditionally
    // (from offset 0 when the dword lies outside the text) and masked after,
    // so the 24 loads overlap.  A dword holding byte n-1 is read whole: the
    // text is 16-byte aligned, so it lies in the same page as that byte.
#pragma unroll
    for (int q = 0; q < 24; ++q) {
      const int64_t addr = base - 16 + 4 * q;
      const bool in = addr >= 0 && uint64_t(addr) < n;
      const uint32_t raw = *reinterpret_cast<const uint32_t *>(text + (in ? addr : 0));
      const int64_t left = int64_t(n) - addr;  // bytes of the dword inside the text
      const uint32_t keep = !in ? 0u : (left >= 4 ? ~0u : ((1u << (8 * left)) - 1u));
      win.w[q] = raw & keep;
    }
  }
}

// ---------------------------------------------------------------------------
// Per-word masks.
// ---------------------------------------------------------------------------
struct WordMasks {
  uint64_t valid;  // byte index < n
  uint64_t lead;   // first byte of a character (stray bytes count as their own char)
  uint64_t L;      // \p{L}
  uint64_t N;      // \p{N}
  uint64_t WS;     // \s (White_Space)
  uint64_t CR;     // \r or \n
  uint64_t SP;     // U+0020
  uint64_t AP;     // U+0027
  uint64_t M;      // \p{M}
  uint64_t LU;     // Lu, Lt
  uint64_t LL;     // Ll
  uint64_t LB;     // Lm, Lo
  // ASCII byte patterns for the contraction clause: s d m t / l / v / e / r
  // (either case), and the two bytes of U+017F
  uint64_t c_sdmt, c_l, c_v, c_e, c_r, c_ls0, c_ls1;
  uint64_t na;     // bytes >= 0x80
  uint32_t err;    // first invalid-sequence byte in [0,64), or 64
};

// Segment starts at window indices -8..119 of a lane (bit j <-> index j-8),
// found by binary search in seg_off[0..n_seg].  Also returns the index of the
// last non-empty... segment containing byte `base` (or the first segment).
__device__ __forceinline__ void segment_marks(const uint64_t *__restrict__ seg_off, uint32_t n_seg,
                                              int64_t base, uint64_t &lo, uint64_t &hi,
                                              uint32_t &seg_at_base) {
  lo = hi = 0;
  // first s with seg_off[s] >= base - 8
  const int64_t from = base - 8;
  uint32_t a = 0, b = n_seg;  // search in [0, n_seg)
  while (a < b) {
    uint32_t mid = (a + b) >> 1;
    if (int64_t(seg_off[mid]) < from) a = mid + 1;
    else b = mid;
  }
  for (uint32_t s = a; s < n_seg; ++s) {
    const int64_t o = int64_t(seg_off[s]);
    if (o >= base + 120) break;
    const int j = int(o - from);
    if (j < 64) lo |= bit(j);
    else hi |= bit(j - 64);
  }
  // segment containing byte base: last s with seg_off[s] <= base
  a = 0;
  b = n_seg;
  while (a < b) {
    uint32_t mid = (a + b) >> 1;
    if (int64_t(seg_off[mid]) <= base) a = mid + 1;
    else b = mid;
  }
  seg_at_base = a > 0 ? a - 1 : 0;
}

// Position of the k-th (from 0) set bit of x, for k < popcount(x): a binary
// search over halves by population count.
__device__ __forceinline__ int nth_set_bit(uint64_t x, uint32_t k) {
  int pos = 0;
#pragma unroll
  for (int wdt = 32; wdt >= 1; wdt >>= 1) {
    const uint32_t lo = uint32_t(__popcll(x & ((uint64_t(1) << wdt) - 1)));
    if (k >= lo) {
      k -= lo;
      x >>= wdt;
      pos += wdt;
    }
  }
  return pos;
}

// ---------------------------------------------------------------------------
// Per-lane folds over short runs of per-tile values (the tile scans folded
// into the per-tile kernels).  Loads are issued eight at a time before any is
// used, so a run of up to 32 values costs four memory round trips, not 32.
// ---------------------------------------------------------------------------
constexpr uint32_t FOLD_BATCH = 8;

// f(q, p[q]) for q = q0, q0 + 1, ..., q1 - 1, in that order
template <typename V, typename F>
__device__ __forceinline__ void fold_run(const V *p, uint32_t q0, uint32_t q1, F f) {
  for (uint32_t q = q0; q < q1; q += FOLD_BATCH) {
    V v[FOLD_BATCH];
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) v[j] = (q + j < q1) ? p[q + j] : V(0);
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j)
      if (q + j < q1) f(q + j, v[j]);
  }
}

// f(q, p[q]) for q = q1 - 1, q1 - 2, ..., q0, in that order
template <typename V, typename F>
__device__ __forceinline__ void fold_run_rev(const V *p, uint32_t q0, uint32_t q1, F f) {
  for (uint32_t q = q1; q > q0; q -= min(q - q0, FOLD_BATCH)) {
    V v[FOLD_BATCH];
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) v[j] = (q - q0 > j) ? p[q - 1 - j] : V(0);
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j)
      if (q - q0 > j) f(q - 1 - j, v[j]);
  }
}

// f(q, p[q]) for q = q0, q0 + step, ... below q1
template <typename V, typename F>
__device__ __forceinline__ void fold_strided(const V *p, uint32_t q0, uint32_t q1, uint32_t step, F f) {
  for (uint32_t q = q0; q < q1; q += FOLD_BATCH * step) {
    V v[FOLD_BATCH];
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) v[j] = (q + j * step < q1) ? p[q + j * step] : V(0);
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j)
      if (q + j * step < q1) f(q + j * step, v[j]);
  }
}

}  // namespace bbpe
