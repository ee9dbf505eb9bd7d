// Classification of one 64-byte word into per-class bitmasks (gfx950).
//
// ASCII bytes are classified four at a time with SWAR range tests on 32-bit
// words (the high bit of each byte lane carries the result), so the common
// all-ASCII word needs no per-byte branches.  Bytes >= 0x80 are handled by a
// slow path that decodes only the multi-byte characters: the wave lists the
// leads of all its words and its 64 lanes share them out, each validating
// UTF-8 and looking up the code point's class for every 64th lead, eight at
// a time so that their loads overlap.  The result is stored per word and
// read back by later passes over the same text.
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

// What the multi-byte characters of a word add to its masks.  Computed once
// per call (by the first front-end kernel, which stores it for every word
// holding a byte >= 0x80) and read back by the later ones.
struct SlowMasks {
  uint64_t LU, LL, LB, N, WS, M, lead, ls0, ls1, err;
};

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

// The wave's multi-byte characters are decoded by all 64 lanes together:
// their lead positions go to a list, each lane decodes every 64th entry, and
// a per-byte code array carries the results back to the words.  The stage
// also holds the wave's bytes and the first class-table stage for the Basic
// Multilingual Plane (code points >> 8 below 256).
constexpr uint32_t LEAD_LIST = 1024;
struct SlowStage {
  uint64_t seg[65];  // segment starts at stage positions (bit q & 63 of seg[q >> 6])
  uint4 bytes[STAGE_BYTES / 16];
  uint4 code[STAGE_BYTES / 16];  // per stage byte: what the decoder found there
  uint16_t u1[256];
  uint32_t ls;                   // some character decoded is U+017F
  union {
    uint16_t list[LEAD_LIST];  // stage positions of the leads
    struct {                   // (before that) the segment-start search:
      uint64_t sm[2][64];      // each lane's window bits
      uint32_t sh[64];         // segment starts counted from each lane on
    } sq;
  };
};

// Per-byte codes of the wave decoder: on every byte of a valid character its
// class code plus one (bits 0..2; 0 where no valid character claims the
// byte), and on the lead and the second byte of U+017F bits 3 and 4.
constexpr uint32_t CODE_LS0 = 0x08, CODE_LS1 = 0x10;

// bits [i, i + len) of a 128-bit mask held as two words, i < 64, len <= 4
__device__ __forceinline__ bool any_in128(uint64_t w0, uint64_t w1, int i, int len) {
  const uint64_t m0 = bit_range(i, len);
  const int over = i + len - 64;
  const uint64_t m1 = over > 0 ? (bit(over) - 1) : 0;
  return ((w0 & m0) | (w1 & m1)) != 0;
}

// Decodes list entries [0, count) of the stage (every 64th from this lane,
// eight at a time: their byte reads, then their class-table reads, issued
// together) and writes their codes.  segs: the stage holds a segment start
// (none may fall on a continuation byte).
__device__ __forceinline__ void decode_listed(const DevTables &T, SlowStage &st, uint32_t count, int lane,
                                              bool segs) {
  const uint32_t *b32 = reinterpret_cast<const uint32_t *>(st.bytes);
  uint8_t *code = reinterpret_cast<uint8_t *>(st.code);
  for (uint32_t g0 = 0; g0 < count; g0 += 64u * 8u) {
    constexpr int K = 8;
    uint32_t q[K], v[K], cp[K], blk[K], cls[K];
    int len[K];
    bool ok[K], has[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint32_t g = g0 + uint32_t(lane) + 64u * uint32_t(k);
      has[k] = g < count;
      q[k] = st.list[has[k] ? g : 0u];
    }
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = __builtin_amdgcn_alignbyte(b32[(q[k] >> 2) + 1], b32[q[k] >> 2], q[k] & 3u);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint32_t w = v[k], b0 = w & 0xFFu;
      const int Ln = b0 < 0xC2u ? 0 : (b0 < 0xE0u ? 2 : (b0 < 0xF0u ? 3 : (b0 < 0xF5u ? 4 : 0)));
      const uint32_t cm = Ln == 2 ? 0xC000u : (Ln == 3 ? 0xC0C000u : 0xC0C0C000u);
      bool good = has[k] && Ln >= 2 && (w & cm) == (cm & 0x80808080u);
      const uint32_t f1 = (w >> 8) & 0x3Fu, f2 = (w >> 16) & 0x3Fu, f3 = (w >> 24) & 0x3Fu;
      const uint32_t c = Ln == 2 ? (((b0 & 0x1Fu) << 6) | f1)
                       : Ln == 3 ? (((b0 & 0x0Fu) << 12) | (f1 << 6) | f2)
                                 : (((b0 & 0x07u) << 18) | (f1 << 12) | (f2 << 6) | f3);
      if (Ln == 3 && c < 0x800) good = false;
      if (Ln == 4 && (c < 0x10000 || c > 0x10FFFF)) good = false;
      if (c >= 0xD800 && c <= 0xDFFF) good = false;
      // no segment starts at a continuation byte (q + Ln - 1 < 64 * 65)
      if (segs && good) {
        const uint32_t e = q[k] >> 6;
        const int b = int(q[k] & 63u);
        const uint64_t s1 = (b + Ln > 64) ? st.seg[e + 1] : 0ull;
        good = !any_in128(st.seg[e], s1, b + 1, Ln - 1);
      }
      cp[k] = c;
      len[k] = Ln;
      ok[k] = good;
    }
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
    for (int k = 0; k < K; ++k) cls[k] = T.uni2[ok[k] ? blk[k] * 256u + (cp[k] & 0xFFu) : 0u];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (!ok[k]) continue;  // an invalid lead keeps code 0
      const uint32_t cv = (cls[k] & 7u) + 1u;
      const bool ls = cp[k] == 0x17F;
      code[q[k]] = uint8_t(cv | (ls ? CODE_LS0 : 0u));
      code[q[k] + 1] = uint8_t(cv | (ls ? CODE_LS1 : 0u));
      if (len[k] > 2) code[q[k] + 2] = uint8_t(cv);
      if (len[k] > 3) code[q[k] + 3] = uint8_t(cv);
      if (ls) st.ls = 1;
    }
  }
}

// The multi-byte part of every lane's word, the wave's characters decoded by
// all lanes together.  Every lane of the wave calls this (lane = threadIdx.x,
// consecutive lanes at consecutive words); r is set for lanes whose word
// holds a byte >= 0x80.  Stages the wave's bytes and the first class-table
// stage in st.
__device__ __forceinline__ void classify_slow_wave(const DevTables &T, const Window &win, int64_t base,
                                                   uint64_t seg_lo, uint64_t seg_hi, uint64_t hi2,
                                                   uint64_t non, uint64_t valid, SlowStage &st, int lane,
                                                   SlowMasks &r) {
  const uint2 u1v = reinterpret_cast<const uint2 *>(T.uni1)[lane];  // stored once it is needed
  stage_window(st.bytes, win, lane);
  const uint64_t leads = hi2 & valid;
  // a character that began up to three bytes before lane 0's word (later
  // lanes' such characters start in the previous lane's word)
  int pre = -1;
  if (lane == 0 && !(hi2 & 1) && (non & 1)) {
    int kf = 0;
    if ((win.at(-1) & 0xC0u) != 0x80u) kf = 1;
    else if ((win.at(-2) & 0xC0u) != 0x80u) kf = 2;
    else if ((win.at(-3) & 0xC0u) != 0x80u) kf = 3;
    if (kf > 0 && base - kf >= 0 && win.at(-kf) >= 0xC0u) pre = 16 - kf;
  }
  const uint32_t cnt = uint32_t(__popcll(leads)) + (pre >= 0 ? 1u : 0u);
  const uint32_t incl = wave_incl_sum(cnt, lane);
  const uint32_t total = __shfl(incl, 63, 64);
  for (uint32_t j = uint32_t(lane); j < STAGE_BYTES / 16; j += 64) st.code[j] = uint4{0, 0, 0, 0};
  // stage positions 64(l+1) .. 64(l+2)-1 are window indices 56..119 of lane l
  const uint64_t sg = (seg_lo >> 56) | (seg_hi << 8);
  st.seg[lane + 1] = sg;
  const uint64_t sg0 = lane == 0 ? (seg_lo << 8) : 0ull;
  if (lane == 0) {
    st.seg[0] = sg0;
    st.ls = 0;
  }
  const bool segs = __ballot((sg | sg0) != 0) != 0;
  __syncthreads();
  const uint32_t w0 = 16u + 64u * uint32_t(lane);  // the word's first byte in the stage
  if (total <= LEAD_LIST) {
    // the word's leads from both halves at once (the list's order is free)
    uint32_t k = incl - cnt;
    if (pre >= 0) st.list[k++] = uint16_t(pre);
    uint32_t xl = uint32_t(leads), xh = uint32_t(leads >> 32);
    uint32_t kh = k + uint32_t(__popc(xl));
    while (xl | xh) {
      if (xl) {
        st.list[k++] = uint16_t(w0 + uint32_t(__ffs(xl) - 1));
        xl &= xl - 1;
      }
      if (xh) {
        st.list[kh++] = uint16_t(w0 + 32u + uint32_t(__ffs(xh) - 1));
        xh &= xh - 1;
      }
    }
    reinterpret_cast<uint2 *>(st.u1)[lane] = u1v;
    __syncthreads();
    decode_listed(T, st, total, lane, segs);
    __syncthreads();
  } else {
    // in pieces of LEAD_LIST entries
    for (uint32_t c0 = 0; c0 < total; c0 += LEAD_LIST) {
      const uint32_t c1 = min(total, c0 + LEAD_LIST);
      uint32_t k = incl - cnt;
      if (pre >= 0) {
        if (k >= c0 && k < c1) st.list[k - c0] = uint16_t(pre);
        ++k;
      }
      for (uint64_t x = leads; x && k < c1; x &= x - 1, ++k)
        if (k >= c0) st.list[k - c0] = uint16_t(w0 + uint32_t(__ffsll(static_cast<unsigned long long>(x)) - 1));
      if (c0 == 0) reinterpret_cast<uint2 *>(st.u1)[lane] = u1v;
      __syncthreads();
      decode_listed(T, st, c1 - c0, lane, segs);
      __syncthreads();
    }
  }
  if (!non) return;
  // this word's 64 codes, one bit per byte and field
  const uint4 *cw = st.code + 1 + 4 * lane;
  uint64_t p0 = 0, p1 = 0, p2 = 0;
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    const uint4 c4 = cw[qd];
    const uint32_t f4[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sh = 4 * (4 * qd + j);
      p0 |= gather4((f4[j] << 7) & 0x80808080u) << sh;
      p1 |= gather4((f4[j] << 6) & 0x80808080u) << sh;
      p2 |= gather4((f4[j] << 5) & 0x80808080u) << sh;
    }
  }
  uint64_t l0 = 0, l1 = 0;
  if (st.ls) {  // (wave-uniform)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const uint4 c4 = cw[qd];
      const uint32_t f4[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int sh = 4 * (4 * qd + j);
        l0 |= gather4((f4[j] << 4) & 0x80808080u) << sh;
        l1 |= gather4((f4[j] << 3) & 0x80808080u) << sh;
      }
    }
  }
  // class code plus one: 1 other, 2 Lu/Lt, 3 Ll, 4 Lm/Lo, 5 N, 6 White_Space, 7 M
  r = SlowMasks{0, 0, 0, 0, 0, 0, 0, 0, 0, 64};
  r.LU = ~p0 & p1 & ~p2;
  r.LL = p0 & p1 & ~p2;
  r.LB = ~p0 & ~p1 & p2;
  r.N = p0 & ~p1 & p2;
  r.WS = ~p0 & p1 & p2;
  r.M = p0 & p1 & p2;
  const uint64_t claimed = p0 | p1 | p2;
  const uint64_t stray = non & ~hi2 & ~claimed;  // continuation bytes no character claims
  const uint64_t errs = (leads & ~claimed) | stray;
  r.err = errs ? uint64_t(__ffsll(static_cast<unsigned long long>(errs)) - 1) : 64u;
  r.lead = leads | stray;
  r.ls0 = l0;
  r.ls1 = l1;
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
                                              SlowStage *st) {
  m.valid = 0;
  if (base >= 0 && uint64_t(base) < n) {
    const uint64_t left = n - uint64_t(base);
    m.valid = left >= 64 ? ~uint64_t(0) : (bit(int(left)) - 1);
  }
  m.lead = m.L = m.N = m.WS = m.CR = m.SP = m.AP = m.M = m.LU = m.LL = m.LB = 0;
  m.c_sdmt = m.c_l = m.c_v = m.c_e = m.c_r = m.c_ls0 = m.c_ls1 = 0;
  m.err = 64;
  m.na = 0;
  // (the decoding kernel goes on with every lane: the wave decodes together;
  // a word outside the text has a zero window and no valid byte)
  if (!COMPUTE && !m.valid) return;

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
  SlowMasks r;
  bool have = false;
  if (COMPUTE) {
    if (__ballot(non != 0)) {  // wave-uniform: every lane takes part
      classify_slow_wave(T, win, base, seg_lo, seg_hi, hi2, non, m.valid, *st, int(threadIdx.x), r);
      have = non != 0;
      if (have && slow_out) {
        ulonglong2 *q = reinterpret_cast<ulonglong2 *>(slow_out);
        q[0] = ulonglong2{r.LU, r.LL};
        q[1] = ulonglong2{r.LB, r.N};
        q[2] = ulonglong2{r.WS, r.M};
        q[3] = ulonglong2{r.lead, r.ls0};
        q[4] = ulonglong2{r.ls1, r.err};
      }
    }
  } else if (non) {
    const ulonglong2 *q = reinterpret_cast<const ulonglong2 *>(slow_in);
    const ulonglong2 v0 = q[0], v1 = q[1], v2 = q[2], v3 = q[3], v4 = q[4];
    r = SlowMasks{v0.x, v0.y, v1.x, v1.y, v2.x, v2.y, v3.x, v3.y, v4.x, v4.y};
    have = true;
  }
  if (have) {
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
