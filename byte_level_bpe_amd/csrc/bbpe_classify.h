// Classification of one 64-byte word into per-class bitmasks (gfx950).
//
// ASCII bytes are classified four at a time with SWAR range tests on 32-bit
// words (the high bit of each byte lane carries the result), so the common
// all-ASCII word needs no per-byte branches.  Bytes >= 0x80 are handled by a
// slow path that decodes only the multi-byte characters, reading their bytes
// from the text, validates UTF-8 and looks up the code point's class, eight
// characters at a time so that their loads overlap; its result is stored
// per word and read back by later passes over the same text.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bbpe_device.h"

namespace bbpe {

// For four bytes < 0x80 packed in d: 0x80 in every byte lane whose byte is >= lo (lo <= 0x80).
__device__ __forceinline__ uint32_t swar_ge(uint32_t d, uint32_t lo) {
  return (d + (0x80808080u - lo * 0x01010101u)) & 0x80808080u;
}
__device__ __forceinline__ uint32_t swar_in(uint32_t d, uint32_t lo, uint32_t hi) {
  return swar_ge(d, lo) & ~swar_ge(d, hi + 1);
}
__device__ __forceinline__ uint32_t swar_eq(uint32_t d, uint32_t c) { return swar_in(d, c, c); }
// the four byte-lane flags (bit 7 of each byte) as a 4-bit value
__device__ __forceinline__ uint64_t gather4(uint32_t f) {
  return uint64_t((((f >> 7) * 0x00204081u) >> 21) & 0xFu);
}

// Bits [i, i+len) of a 64-bit mask, clipped to [0, 64).
__device__ __forceinline__ uint64_t bit_range(int i, int len) {
  const int e = min(64, i + len);
  if (e <= i) return 0;
  const uint64_t hi = (e == 64) ? ~uint64_t(0) : (bit(e) - 1);
  return hi & ~(bit(i) - 1);
}

__device__ __forceinline__ bool seg_start_at(uint64_t seg_lo, uint64_t seg_hi, int k) {
  const int s = k + 8;  // window index k -> segment-mask bit k + 8
  if (s < 0 || s >= 128) return false;
  return s < 64 ? ((seg_lo >> s) & 1) : ((seg_hi >> (s - 64)) & 1);
}

// What the multi-byte characters of a word add to its masks.  Computed once
// per call (by the first front-end kernel, which stores it for every word
// holding a byte >= 0x80) and read back by the later ones.
struct SlowMasks {
  uint64_t LU, LL, LB, N, WS, M, lead, ls0, ls1, err;
};

__device__ __forceinline__ void add_class(SlowMasks &r, uint32_t cls, uint64_t bits) {
  r.LU |= (cls == CC_LU) ? bits : 0;
  r.LL |= (cls == CC_LL) ? bits : 0;
  r.LB |= (cls == CC_LO) ? bits : 0;
  r.N |= (cls == CC_N) ? bits : 0;
  r.WS |= (cls == CC_WS) ? bits : 0;
  r.M |= (cls == CC_M) ? bits : 0;
}

// The text bytes of one wave's 64 windows in LDS: bytes [lo, lo + 4128),
// where lo is 16 bytes before lane 0's word (the windows hold 0 outside the
// text), so that per-character byte reads go to LDS instead of memory.
constexpr uint32_t STAGE_BYTES = 64 * 64 + 32;

// Every lane of the wave calls this with its own window (lane = threadIdx.x
// < 64, consecutive lanes at consecutive words); no barrier.
__device__ __forceinline__ void stage_window(uint4 *bytes, const Window &win, int lane) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    bytes[1 + 4 * lane + q] = uint4{win.w[4 + 4 * q], win.w[5 + 4 * q], win.w[6 + 4 * q], win.w[7 + 4 * q]};
  if (lane == 0) bytes[0] = uint4{win.w[0], win.w[1], win.w[2], win.w[3]};
  if (lane == 63) bytes[STAGE_BYTES / 16 - 1] = uint4{win.w[20], win.w[21], win.w[22], win.w[23]};
}

// byte p of the text from a staged tile (p in [lo, lo + STAGE_BYTES))
__device__ __forceinline__ uint32_t staged_byte(const uint4 *bytes, int64_t lo, int64_t p) {
  return reinterpret_cast<const uint8_t *>(bytes)[p - lo];
}

// The staged bytes and the first stage of the class table for the Basic
// Multilingual Plane (code points >> 8 below 256), for the multi-byte decoder.
struct SlowStage {
  uint4 bytes[STAGE_BYTES / 16];
  uint16_t u1[256];
};

__device__ __forceinline__ void stage_fill(SlowStage &st, const DevTables &T, const Window &win, int lane) {
  const uint2 u = reinterpret_cast<const uint2 *>(T.uni1)[lane];
  reinterpret_cast<uint2 *>(st.u1)[lane] = u;
  stage_window(st.bytes, win, lane);
  __syncthreads();
}

// The multi-byte characters of the word at base: `hi2` marks its bytes >=
// 0xC0, `non` its bytes >= 0x80.  Leads are decoded eight at a time with all
// their byte loads, then all their class-table loads, issued together.
__device__ __forceinline__ void classify_slow(const DevTables &T, const uint8_t *__restrict__ text,
                                              const Window &win, int64_t base, uint64_t n,
                                              uint64_t seg_lo, uint64_t seg_hi, uint64_t hi2,
                                              uint64_t non, uint64_t valid, const SlowStage &st,
                                              int64_t lo, SlowMasks &r) {
  r = SlowMasks{0, 0, 0, 0, 0, 0, 0, 0, 0, 64};
  uint64_t covered = 0;
  uint32_t err = 64;
  // a character that began up to three bytes before the word
  if (!(hi2 & 1) && (non & 1)) {
    int kf = 0;
    if ((win.at(-1) & 0xC0u) != 0x80u) kf = 1;
    else if ((win.at(-2) & 0xC0u) != 0x80u) kf = 2;
    else if ((win.at(-3) & 0xC0u) != 0x80u) kf = 3;
    if (kf > 0 && base - kf >= 0) {
      // its bytes from the window (fixed indices, selected by kf)
      uint32_t b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = kf == 1 ? win.at(j - 1) : (kf == 2 ? win.at(j - 2) : win.at(j - 3));
      const int len = utf8_len(b[0]);
      bool ok = len >= 2 && uint64_t(base - kf) + uint64_t(len) <= n;
      uint32_t cp = b[0] & (0x7Fu >> len);
#pragma unroll
      for (int j = 1; j < 4; ++j) {
        const bool in = j < len;
        ok = ok && (!in || (((b[j] & 0xC0u) == 0x80u) && !seg_start_at(seg_lo, seg_hi, j - kf)));
        cp = in ? ((cp << 6) | (b[j] & 0x3Fu)) : cp;
      }
      if (len == 3 && cp < 0x800) ok = false;
      if (len == 4 && (cp < 0x10000 || cp > 0x10FFFF)) ok = false;
      if (cp >= 0xD800 && cp <= 0xDFFF) ok = false;
      if (ok && len > kf) {
        const uint32_t blk = cp <= 0xFFFFu ? uint32_t(st.u1[cp >> 8]) : uint32_t(T.uni1[cp >> 8]);
        const uint64_t bits = bit_range(0, len - kf);
        covered |= bits;
        add_class(r, T.uni2[blk * 256u + (cp & 0xFFu)], bits);
        if (cp == 0x17F) r.ls1 |= 1;  // its second byte
      }
    }
  }
  // invalid lead bytes (C0, C1, F5..FF) are >= 0xC0 too and fail to decode
  uint64_t leads = hi2 & valid;
  uint64_t lead = 0;
  // segment starts at word positions 0..63, and 64..66 in bits 0..2
  const uint64_t segw = (seg_lo >> 8) | (seg_hi << 56);
  const uint32_t segx = uint32_t(seg_hi >> 8) & 7u;
  // class code planes of the batch loop's characters (bit b of the code)
  uint64_t pl0 = 0, pl1 = 0, pl2 = 0;
  const uint32_t *b32 = reinterpret_cast<const uint32_t *>(st.bytes);
  const uint32_t a0 = uint32_t(base - lo);  // the word's first byte in the stage
  while (leads) {
    constexpr int K = 8;
    int ii[K];
    uint32_t v[K];  // the four bytes from each lead, little endian
#pragma unroll
    for (int k = 0; k < K; ++k) {
      ii[k] = __ffsll(static_cast<unsigned long long>(leads)) - 1;  // -1 once none are left
      leads &= leads - 1;
      const uint32_t ad = uint32_t(int(a0) + ii[k]);
      v[k] = __builtin_amdgcn_alignbyte(b32[(ad >> 2) + 1], b32[ad >> 2], ad & 3u);
    }
    uint32_t cp[K], blk[K];
    int len[K];
    bool ok[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint32_t w = v[k], b0 = w & 0xFFu;
      const int Ln = b0 < 0xC2u ? 0 : (b0 < 0xE0u ? 2 : (b0 < 0xF0u ? 3 : (b0 < 0xF5u ? 4 : 0)));
      // continuation bytes 1 .. Ln-1 of the form 10xxxxxx
      const uint32_t cm = Ln == 2 ? 0xC000u : (Ln == 3 ? 0xC0C000u : 0xC0C0C000u);
      bool good = ii[k] >= 0 && Ln >= 2 && (w & cm) == (cm & 0x80808080u);
      const uint32_t f1 = (w >> 8) & 0x3Fu, f2 = (w >> 16) & 0x3Fu, f3 = (w >> 24) & 0x3Fu;
      const uint32_t c = Ln == 2 ? (((b0 & 0x1Fu) << 6) | f1)
                       : Ln == 3 ? (((b0 & 0x0Fu) << 12) | (f1 << 6) | f2)
                                 : (((b0 & 0x07u) << 18) | (f1 << 12) | (f2 << 6) | f3);
      if (Ln == 3 && c < 0x800) good = false;
      if (Ln == 4 && (c < 0x10000 || c > 0x10FFFF)) good = false;
      if (c >= 0xD800 && c <= 0xDFFF) good = false;
      // no segment starts at a continuation byte
      const int i = ii[k] < 0 ? 0 : ii[k];
      const uint64_t cont = bit_range(i + 1, Ln - 1);
      const int ext = i + Ln - 64;  // continuation bytes past the word
      const bool segbad = (segw & cont) != 0 || (ext > 0 && (segx & ((1u << ext) - 1u)) != 0);
      cp[k] = c;
      len[k] = Ln;
      ok[k] = good && !segbad;
    }
    // second-stage loads issued unconditionally (index 0 when unused: a load
    // under a condition is waited for on its own); the first stage is read
    // from LDS, and from memory only for code points beyond U+FFFF
    uint32_t cls[K];
    bool astral = false;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      blk[k] = st.u1[ok[k] ? ((cp[k] >> 8) & 0xFFu) : 0u];
      astral = astral || (ok[k] && cp[k] > 0xFFFFu);
    }
    if (astral) {
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (ok[k] && cp[k] > 0xFFFFu) blk[k] = T.uni1[cp[k] >> 8];
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint32_t c = T.uni2[ok[k] ? blk[k] * 256u + (cp[k] & 0xFFu) : 0u];
      cls[k] = ok[k] ? c : 0u;
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = ii[k];
      if (i < 0) continue;
      lead |= bit(i);
      if (!ok[k]) {
        err = min(err, uint32_t(i));
        continue;
      }
      const uint64_t bits = bit_range(i, len[k]);
      covered |= bits & ~bit(i);
      pl0 |= (cls[k] & 1u) ? bits : 0;
      pl1 |= (cls[k] & 2u) ? bits : 0;
      pl2 |= (cls[k] & 4u) ? bits : 0;
      if (cp[k] == 0x17F) {
        r.ls0 |= bit(i);
        if (i + 1 < 64) r.ls1 |= bit(i + 1);
      }
    }
  }
  // planes to class masks (class codes 1..6; 0, "other", sets no plane)
  r.LU |= pl0 & ~pl1 & ~pl2;
  r.LL |= ~pl0 & pl1 & ~pl2;
  r.LB |= pl0 & pl1 & ~pl2;
  r.N |= ~pl0 & ~pl1 & pl2;
  r.WS |= pl0 & ~pl1 & pl2;
  r.M |= ~pl0 & pl1 & pl2;
  // continuation bytes that no valid character claims are errors; they
  // count as characters of their own (class "other")
  const uint64_t cont = non & ~hi2;
  const uint64_t stray = cont & ~covered;
  if (stray) err = min(err, uint32_t(__ffsll(static_cast<unsigned long long>(stray)) - 1));
  r.lead = lead | stray;
  r.err = err;
}

// Classify the 64 bytes of the word at text offset base (window = bytes
// [base-16, base+80)).  seg_lo/seg_hi: segment starts at window indices
// -8..119 (bit j <-> index j-8).  COMPUTE: the multi-byte part is computed
// (and stored to slow_out when given); else it is read from slow_in, the
// word's stored record (kernels after the first never decode, which keeps
// the decoder's registers out of them).
template <bool COMPUTE>
__device__ __forceinline__ void classify_word(const DevTables &T, const uint8_t *__restrict__ text,
                                              const Window &win, int64_t base, uint64_t n,
                                              uint64_t seg_lo, uint64_t seg_hi, WordMasks &m,
                                              const uint64_t *slow_in, uint64_t *slow_out,
                                              const SlowStage *st, int64_t lo) {
  m.valid = 0;
  if (base >= 0 && uint64_t(base) < n) {
    const uint64_t left = n - uint64_t(base);
    m.valid = left >= 64 ? ~uint64_t(0) : (bit(int(left)) - 1);
  }
  m.lead = m.L = m.N = m.WS = m.CR = m.SP = m.AP = m.M = m.LU = m.LL = m.LB = 0;
  m.c_sdmt = m.c_l = m.c_v = m.c_e = m.c_r = m.c_ls0 = m.c_ls1 = 0;
  m.err = 64;
  m.na = 0;
  if (!m.valid) return;

  uint64_t asc = 0, hi2 = 0;  // ASCII bytes; bytes >= 0xC0 (lead bytes of multi-byte chars)
  uint32_t ap_near = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const uint32_t raw = win.w[4 + q];
    const uint32_t a4 = ~raw & 0x80808080u;
    // with bit 7 cleared no byte lane can carry into the next one; the
    // results for non-ASCII lanes are masked off by a4
    const uint32_t d = raw & 0x7F7F7F7Fu;
    const int sh = 4 * q;
    asc |= gather4(a4) << sh;
    hi2 |= gather4(raw & (raw << 1) & 0x80808080u) << sh;
    m.LU |= gather4(swar_in(d, 0x41, 0x5A) & a4) << sh;
    m.LL |= gather4(swar_in(d, 0x61, 0x7A) & a4) << sh;
    m.N |= gather4(swar_in(d, 0x30, 0x39) & a4) << sh;
    m.WS |= gather4((swar_in(d, 9, 13) | swar_eq(d, 32)) & a4) << sh;
    m.CR |= gather4((swar_eq(d, 10) | swar_eq(d, 13)) & a4) << sh;
    m.SP |= gather4(swar_eq(d, 32) & a4) << sh;
    const uint32_t ap = swar_eq(d, 39) & a4;
    m.AP |= gather4(ap) << sh;
    ap_near |= ap;
  }
  {  // apostrophes in the two bytes before the word also look into it
    const uint32_t raw = win.w[3];
    ap_near |= swar_eq(raw & 0x7F7F7F7Fu, 39) & ~raw & 0x80800000u;
  }
  if (ap_near) {
    // letters a contraction may consist of: s d m t l v e r, either case
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t raw = win.w[4 + q];
      const uint32_t a4 = ~raw & 0x80808080u;
      const uint32_t lc = (raw & 0x7F7F7F7Fu) | 0x20202020u;
      const int sh = 4 * q;
      m.c_sdmt |= gather4((swar_eq(lc, 's') | swar_eq(lc, 'd') | swar_eq(lc, 'm') | swar_eq(lc, 't')) & a4) << sh;
      m.c_l |= gather4(swar_eq(lc, 'l') & a4) << sh;
      m.c_v |= gather4(swar_eq(lc, 'v') & a4) << sh;
      m.c_e |= gather4(swar_eq(lc, 'e') & a4) << sh;
      m.c_r |= gather4(swar_eq(lc, 'r') & a4) << sh;
    }
  }
  uint64_t lead = asc;

  const uint64_t non = ~asc & m.valid;
  m.na = non;
  if (non) {
    SlowMasks r;
    if (!COMPUTE) {
      const ulonglong2 *q = reinterpret_cast<const ulonglong2 *>(slow_in);
      const ulonglong2 v0 = q[0], v1 = q[1], v2 = q[2], v3 = q[3], v4 = q[4];
      r = SlowMasks{v0.x, v0.y, v1.x, v1.y, v2.x, v2.y, v3.x, v3.y, v4.x, v4.y};
    } else {
      classify_slow(T, text, win, base, n, seg_lo, seg_hi, hi2, non, m.valid, *st, lo, r);
      if (slow_out) {
        ulonglong2 *q = reinterpret_cast<ulonglong2 *>(slow_out);
        q[0] = ulonglong2{r.LU, r.LL};
        q[1] = ulonglong2{r.LB, r.N};
        q[2] = ulonglong2{r.WS, r.M};
        q[3] = ulonglong2{r.lead, r.ls0};
        q[4] = ulonglong2{r.ls1, r.err};
      }
    }
    m.LU |= r.LU;
    m.LL |= r.LL;
    m.LB |= r.LB;
    m.N |= r.N;
    m.WS |= r.WS;
    m.M |= r.M;
    m.c_ls0 |= r.ls0;
    m.c_ls1 |= r.ls1;
    lead |= r.lead;
    m.err = uint32_t(r.err);
  }
  const uint64_t v = m.valid;
  m.L = m.LU | m.LL | m.LB;
  m.lead = lead & v;
  m.L &= v; m.N &= v; m.WS &= v; m.CR &= v; m.SP &= v; m.AP &= v; m.M &= v;
  m.LU &= v; m.LL &= v; m.LB &= v;
  m.c_sdmt &= v; m.c_l &= v; m.c_v &= v; m.c_e &= v; m.c_r &= v; m.c_ls0 &= v; m.c_ls1 &= v;
  if (m.err < 64 && !((v >> m.err) & 1)) m.err = 64;
}

}  // namespace bbpe
