// Split of every span into pre-tokens, as piece-start bits, for the cl100k
// grammar, the o200k-style grammar and the r50k-style grammar (cl100k with
// r50k's digit clause, run by the cl100k kernels).
//
// The printed patterns are applied leftmost-first with possessive
// quantifiers (tiktoken deep-dive page, "The split pattern"; the o200k-style
// letter clause from "r50k, cl100k, o200k").  Rather than running a regex
// engine, each lane derives the match starts of its 64-byte word from class
// bitmasks: whether a match starts at a character depends only on the
// characters a few bytes around it, except for quantities carried along the
// text:
//   * the position of a digit inside its digit run, modulo 3 (digit groups of
//     at most three; not needed by the r50k-style digit clause, whose run
//     is one match, led by a single space before it when there is one);
//   * whether a run of non-CR/LF whitespace reaches a non-space character of
//     the same span (the last CR/LF of a whitespace run ends a match only if
//     the whitespace after it is followed by a non-space character); (both)
//   * cl100k: whether a run of CR/LF characters at the start of a whitespace
//     run was preceded by punctuation (the punctuation clause then swallows
//     those CR/LF characters, and the whitespace clauses restart after them);
//   * o200k-style: the state of an eleven-state automaton over letters, marks and
//     punctuation, which also covers the CR/LF run of the cl100k case (see
//     "o200k-style letter automaton" below).
// The digit phase and the automaton flow left to right, the whitespace
// quantity right to left.  Each lane summarises its word as a transfer
// function on the carried state; functions compose across lanes (wave scans)
// and across tiles (a one-workgroup scan).
#include <hip/hip_runtime.h>

#include "bbpe_classify.h"
#include "bbpe_device.h"
#include "bbpe_kernels.h"
#include "bbpe_machines.h"
#include "bbpe_word.h"

namespace bbpe {

// ---------------------------------------------------------------------------
// Transfer-function encodings.
//   digit phase: states 0,1,2 (index of the last digit in its run, mod 3) and
//                3 (not in a digit run); 4 entries of 2 bits.
//   CR run:      states 0 (none), 1 (CR/LF run that followed punctuation),
//                2 (other CR/LF run); 3 entries of 2 bits.      (cl100k)
//   letter:      the o200k-style automaton, 11 entries of 4 bits.
//   v (RTL):     state = "the non-CR/LF whitespace continuing here ends at a
//                non-space character of the span"; 2 entries of 1 bit.
// A word's or tile's functions are packed in 64 bits (the layout per
// grammar is given with ltr_then below).
// ---------------------------------------------------------------------------
constexpr uint32_t FDIG_ID = 0xE4u;  // 3,2,1,0
constexpr uint32_t FV_ID = 0x2u;     // 1,0
constexpr uint32_t NLET = 11;
constexpr uint64_t FLET_ID = 0xA9876543210ull;
constexpr uint64_t FLET_ONES = 0x11111111111ull;

__device__ __forceinline__ uint32_t fdig_apply(uint32_t f, uint32_t s) { return (f >> (2 * s)) & 3u; }
__device__ __forceinline__ uint32_t flet_apply(uint64_t f, uint32_t s) { return uint32_t(f >> (4 * s)) & 15u; }
__device__ __forceinline__ uint32_t fv_apply(uint32_t f, uint32_t s) { return (f >> s) & 1u; }
// f first, then g
__device__ __forceinline__ uint32_t fdig_then(uint32_t f, uint32_t g) {
  uint32_t h = 0;
#pragma unroll
  for (uint32_t s = 0; s < 4; ++s) h |= fdig_apply(g, fdig_apply(f, s)) << (2 * s);
  return h;
}
__device__ __forceinline__ uint64_t flet_then(uint64_t f, uint64_t g) {
  uint64_t h = 0;
#pragma unroll
  for (uint32_t s = 0; s < NLET; ++s) h |= uint64_t(flet_apply(g, flet_apply(f, s))) << (4 * s);
  return h;
}
__device__ __forceinline__ uint32_t fv_then(uint32_t f, uint32_t g) {
  uint32_t h = 0;
#pragma unroll
  for (uint32_t s = 0; s < 2; ++s) h |= fv_apply(g, fv_apply(f, s)) << s;
  return h;
}

// The left-to-right part of a packed function (digit + CR run or letter)
// and the lookahead function beside it.  cl100k (G == 0): the digit
// function's images of states 0..3 in bytes 0..3 and the CR function's of
// states 0..2 in bytes 4..6, so that composing is one byte permute per
// part; the lookahead function in bits 56-57 (the CR part's unused byte).
// o200k-style (G == 1): 2-bit digit images in bits 0-7, the lookahead in
// bits 8-9, the letter automaton's 4-bit images from bit 16.
template <int G>
__device__ __forceinline__ uint64_t ltr_id() {
  return G == 0 ? 0x0302010003020100ull : (uint64_t(FDIG_ID) | (FLET_ID << 16));
}
template <int G>
__device__ __forceinline__ uint64_t ltr_then(uint64_t f, uint64_t g) {
  if (G == 0) {  // h(s) = g(f(s)): f's bytes select g's (selectors 0..3 pick the second source's bytes)
    const uint32_t lo = __builtin_amdgcn_perm(0u, uint32_t(g), uint32_t(f));
    const uint32_t hi = __builtin_amdgcn_perm(0u, uint32_t(g >> 32), uint32_t(f >> 32));
    return uint64_t(lo) | (uint64_t(hi) << 32);
  }
  return fdig_then(uint32_t(f & 0xFFu), uint32_t(g & 0xFFu)) | (flet_then(f >> 16, g >> 16) << 16);
}
template <int G>
__device__ __forceinline__ uint32_t ltr_apply_dig(uint64_t f, uint32_t s) {
  return G == 0 ? uint32_t(f >> (8 * s)) & 0xFFu : fdig_apply(uint32_t(f & 0xFFu), s);
}
template <int G>
__device__ __forceinline__ uint32_t ltr_apply_x(uint64_t f, uint32_t s) {
  return G == 0 ? uint32_t(f >> (32 + 8 * s)) & 0xFFu : flet_apply(f >> 16, s);
}
// the lookahead part, and the packed function without it
template <int G>
__device__ __forceinline__ uint32_t fn_v(uint64_t f) {
  return uint32_t(f >> (G == 0 ? 56 : 8)) & 3u;
}
template <int G>
__device__ __forceinline__ uint64_t fn_ltr(uint64_t f) {
  return G == 0 ? (f & 0x00FFFFFFFFFFFFFFull) | (uint64_t(3) << 56) : (f & ~uint64_t(0x300));
}
template <int G>
__device__ __forceinline__ uint64_t fn_with_v(uint64_t ltr, uint32_t v) {
  return G == 0 ? (ltr & 0x00FFFFFFFFFFFFFFull) | (uint64_t(v) << 56) : (ltr | (uint64_t(v) << 8));
}

// ---------------------------------------------------------------------------
// o200k-style letter automaton.  The letter clause is an optional prefix
// character P (not CR/LF, letter or digit), then the longest run of U
// characters (Lu Lt Lm Lo M), then the longest run of W characters (Ll Lm
// Lo M), at least one character in all, then an optional contraction; the
// other clauses are cl100k's.  Per character, in text order:
//   F   a match starts at the next character        F1  inside a CR/LF run that
//   F2  inside another CR/LF run                        followed punctuation
//   PS  the last character (O or M) started a match and prefixes letters or
//       starts a punctuation run
//   PSP the last character is a space (prefixes letters or punctuation; a
//       CR/LF after it is whitespace, not the punctuation clause's tail)
//   PW  the last character is other whitespace (prefixes letters only)
//   LU  inside the letters, no W-only (Ll) character yet
//   LW  inside the letters after a W-only character
//   Q   inside a punctuation run
//   C1, C2  one / two characters of a contraction still to come
// Character kinds: X (outside the span), CR, SP (U+0020), WS (other
// whitespace), N, U (Lu Lt), W (Ll), B (Lm Lo), M, O (other), A1 / A2 (an
// apostrophe followed by a one / two character contraction).  Whitespace and
// digit starts are not decided here.
// ---------------------------------------------------------------------------
enum : uint32_t { S_F = 0, S_F1, S_F2, S_PS, S_PSP, S_PW, S_LU, S_LW, S_Q, S_C1, S_C2 };
enum : uint32_t { K_X = 0, K_CR, K_SP, K_WS, K_N, K_U, K_W, K_B, K_M, K_O, K_A1, K_A2, K_COUNT };

struct LetStep {
  uint32_t next;
  bool start;
};
constexpr bool in_set(uint32_t st, uint32_t a, uint32_t b = 99, uint32_t c = 99, uint32_t d = 99) {
  return st == a || st == b || st == c || st == d;
}
constexpr LetStep let_step(uint32_t st, uint32_t k) {
  if (k == K_X || k == K_N) return {S_F, false};
  if (k == K_SP) return {S_PSP, false};
  if (k == K_WS) return {S_PW, false};
  if (k == K_CR) return {in_set(st, S_F1, S_F2) ? st : (in_set(st, S_Q, S_PS) ? S_F1 : S_F2), false};
  if (st == S_C1) return {S_F, false};
  if (st == S_C2) return {S_C1, false};
  const bool pend = in_set(st, S_PS, S_PSP, S_PW);  // a prefix character waits
  if (k == K_U) return {S_LU, !(pend || st == S_LU)};
  if (k == K_W) return {S_LW, !(pend || in_set(st, S_LU, S_LW))};
  if (k == K_B) {
    if (in_set(st, S_LU, S_LW)) return {st, false};
    return {S_LU, !pend};
  }
  if (k == K_M) {
    if (in_set(st, S_LU, S_LW)) return {st, false};
    if (pend) return {S_LU, false};
    if (st == S_Q) return {S_Q, false};
    return {S_PS, true};
  }
  if ((k == K_A1 || k == K_A2) && in_set(st, S_LU, S_LW)) return {k == K_A1 ? S_C1 : S_C2, false};
  // punctuation
  if (in_set(st, S_Q, S_PS, S_PSP)) return {S_Q, false};
  return {S_PS, true};
}
constexpr uint64_t let_table(uint32_t k) {
  uint64_t t = 0;
  for (uint32_t s = 0; s < NLET; ++s) t |= uint64_t(let_step(s, k).next) << (4 * s);
  return t;
}
constexpr uint32_t let_starts(uint32_t k) {
  uint32_t m = 0;
  for (uint32_t s = 0; s < NLET; ++s) m |= uint32_t(let_step(s, k).start) << s;
  return m;
}
struct LetEntry {
  uint64_t t;
  uint32_t sm, pad;
};
__device__ __forceinline__ LetEntry *let_lds() {
  __shared__ LetEntry tab[16];
  return tab;
}
__device__ __forceinline__ void let_kind_switch(uint32_t k, uint64_t &t, uint32_t &sm) {
  switch (k) {
#define BBPE_KIND(K) \
  case K: t = let_table(K); sm = let_starts(K); break;
    BBPE_KIND(K_CR) BBPE_KIND(K_SP) BBPE_KIND(K_WS) BBPE_KIND(K_N) BBPE_KIND(K_U) BBPE_KIND(K_W)
    BBPE_KIND(K_B) BBPE_KIND(K_M) BBPE_KIND(K_O) BBPE_KIND(K_A1) BBPE_KIND(K_A2)
#undef BBPE_KIND
    default: t = let_table(K_X); sm = let_starts(K_X); break;
  }
}
// The per-kind automaton step, read from a 16-entry table in LDS (filled by
// let_fill() at the start of the o200k-style kernels): a lane's kind varies
// per character, and a switch on it became a chain of selects over every
// kind (large workload: split 228 + 485 -> 140 + 329 us with the table).
__device__ __forceinline__ void let_kind(uint32_t k, uint64_t &t, uint32_t &sm) {
  const LetEntry e = let_lds()[k];
  t = e.t;
  sm = e.sm;
}
__device__ __forceinline__ void let_fill() {
  if (threadIdx.x < 16) {
    uint64_t t;
    uint32_t sm;
    let_kind_switch(threadIdx.x, t, sm);
    let_lds()[threadIdx.x] = LetEntry{t, sm, 0};
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Per-word split state.
// ---------------------------------------------------------------------------
struct SplitWord {
  uint64_t SS, SPST, IN, BRK, LD, N_, CR_, NC, WS_, pN, pO, pSP;
  uint64_t K0, K1, K2, K3;   // o200k-style: character kind bit planes
  uint64_t todo;             // o200k-style: bytes the automaton steps on
  uint64_t WstCR;            // o200k-style: CR/LF that begins a whitespace run
  uint64_t static_starts;    // starts that need no carried state
  uint32_t f_dig, f_v, f_cr;
  uint64_t f_let;
};

// Digit-phase and v transfer functions of the word (both grammars).
__device__ __forceinline__ void digit_v_fns(const SplitWord &o, const uint64_t NLD_runstart,
                                            uint32_t &fd, uint32_t &fv) {
  const uint64_t runstart = NLD_runstart;
  if (o.N_ == ~uint64_t(0) && runstart == 0) {
    const uint32_t cnt = uint32_t(__popcll(o.LD)) % 3u;
    fd = 0;
#pragma unroll
    for (uint32_t s = 0; s < 3; ++s) fd |= ((s + cnt) % 3u) << (2 * s);
    fd |= ((cnt + 2u) % 3u) << 6;
  } else {
    fd = digit_phase_out(o.N_, o.N_ & o.LD, runstart) * 0x55u;  // constant function
  }
  const uint64_t prop = o.NC & ~o.BRK;
  if (prop == ~uint64_t(0)) {
    fv = FV_ID;
  } else {
    // v at byte 0 is fixed by the first non-propagating byte
    const int i = __ffsll(static_cast<unsigned long long>(~prop)) - 1;
    const uint64_t b = bit(i);
    const uint32_t v = (o.BRK & b) ? 0u : ((o.WS_ & b) ? 0u : 1u);
    fv = v * 3u;
  }
}

// Everything of the split that does not depend on the carried states, plus
// this word's transfer functions.  Must be called by all 64 lanes.
template <int G>
__device__ __forceinline__ void split_word(const EncodeArgs &a, int64_t w, const WordMasks &m,
                                           SplitWord &o) {
  const bool inrange = w >= 0 && w < int64_t(a.n_words);
  const uint64_t SPST = inrange ? a.ws.spst[w] : 0;
  const uint64_t SPC = inrange ? a.ws.spc[w] : 0;
  // a span also starts right after every special (the first byte outside
  // one after a byte inside), whichever pass chose the special
  const uint64_t SPCq = shfl_up64(SPC, 1);
  const uint64_t SS = (inrange ? a.ws.ss[w] : 0) | (shl(SPC, SPCq, 1) & ~SPC & m.valid);
  const uint64_t IN = m.valid & ~SPC;
  const uint64_t BRK = SS | SPST | ~m.valid;
  const uint64_t L_ = m.L & IN, N_ = m.N & IN, WS_ = m.WS & IN, CR_ = m.CR & IN, SP_ = m.SP & IN;
  const uint64_t O_ = IN & ~(m.L | m.N | m.WS);  // punctuation, marks included
  const uint64_t LD = m.lead & IN;
  const uint64_t CONT = m.valid & ~m.lead;
  const uint64_t INB = IN & ~BRK;
  const uint64_t GL = LD & ~WS_ & ~SS;  // a non-space character that continues the span

  // neighbour words
  const uint64_t Lq = shfl_up64(L_, 1), Nq = shfl_up64(N_, 1), WSq = shfl_up64(WS_, 1);
  const uint64_t CRq = shfl_up64(CR_, 1), SPq = shfl_up64(SP_, 1), Oq = shfl_up64(O_, 1);
  const uint64_t CONTq = shfl_up64(CONT, 1);
  const uint64_t INBn = shfl_down64(INB, 1), sdmtn = shfl_down64(m.c_sdmt, 1);
  const uint64_t ln = shfl_down64(m.c_l, 1), vn = shfl_down64(m.c_v, 1), en = shfl_down64(m.c_e, 1);
  const uint64_t rn = shfl_down64(m.c_r, 1), ls0n = shfl_down64(m.c_ls0, 1);
  const uint64_t ls1n = shfl_down64(m.c_ls1, 1), CONTn = shfl_down64(CONT, 1);
  const uint64_t GLn = shfl_down64(GL, 1);

  // class of the previous byte, within the same span
  const uint64_t pL = shl(L_, Lq, 1) & ~SS, pN = shl(N_, Nq, 1) & ~SS;
  const uint64_t pWS = shl(WS_, WSq, 1) & ~SS, pCR = shl(CR_, CRq, 1) & ~SS;
  const uint64_t pSP = shl(SP_, SPq, 1) & ~SS, pO = shl(O_, Oq, 1) & ~SS;

  // contractions after an apostrophe, inside the span: s d m t (either case,
  // or U+017F) one character on, or ll / ve / re
  const uint64_t nb1 = shr(INB, INBn, 1), nb2 = shr(INB, INBn, 2);
  const uint64_t s1 = shr(m.c_sdmt, sdmtn, 1);
  const uint64_t ls = shr(m.c_ls0, ls0n, 1) & shr(m.c_ls1, ls1n, 2);
  const uint64_t two = (shr(m.c_l, ln, 1) & shr(m.c_l, ln, 2)) | (shr(m.c_v, vn, 1) & shr(m.c_e, en, 2)) |
                       (shr(m.c_r, rn, 1) & shr(m.c_e, en, 2));

  // whitespace: a run starts a match where it begins (cl100k: unless
  // punctuation before it swallowed its leading CR/LF characters, handled by
  // the CR machine; o200k-style: by the automaton); the last non-CR/LF
  // character of a run starts a match when a non-space character of the
  // span follows; the first character after the run's last CR/LF starts one
  // when the rest of the run is followed by a non-space character (the v
  // machine)
  const uint64_t Wst = WS_ & LD & ~pWS;
  const uint64_t NC = WS_ & ~CR_;
  const uint64_t n1 = shr(GL, GLn, 1), kn1 = shr(CONT, CONTn, 1), kn2 = shr(CONT, CONTn, 2);
  const uint64_t kn3 = shr(CONT, CONTn, 3);
  const uint64_t nextGL = n1 | (shr(GL, GLn, 2) & kn1) | (shr(GL, GLn, 3) & kn1 & kn2) |
                          (shr(GL, GLn, 4) & kn1 & kn2 & kn3);
  const uint64_t WL = NC & LD & nextGL;

  o.SS = SS;
  o.SPST = SPST;
  o.IN = IN;
  o.BRK = BRK;
  o.LD = LD;
  o.N_ = N_;
  o.CR_ = CR_;
  o.NC = NC;
  o.WS_ = WS_;
  o.pN = pN;
  o.pO = pO;
  o.pSP = pSP;

  if (G == 0) {
    // punctuation (any non-letter, non-digit, non-space character): a match
    // starts at the first character of a punctuation run unless a single
    // space before it joins the run
    const uint64_t OST = O_ & LD & ~pO & ~pSP;
    // an apostrophe that starts a match and is followed by a contraction:
    // the contraction clause
    const uint64_t APc = m.AP & OST;
    const uint64_t C2M = APc & s1 & nb1;  // the match ends two bytes on
    const uint64_t C3M = APc & nb1 & nb2 & (ls | (two & ~s1));  // three bytes on
    const uint64_t OSTq = shfl_up64(OST, 1), C2q = shfl_up64(C2M, 1), C3q = shfl_up64(C3M, 1);
    const uint64_t R = shl(C2M, C2q, 2) | shl(C3M, C3q, 3);
    const uint64_t k1 = shl(CONT, CONTq, 1), k2 = shl(CONT, CONTq, 2), k3 = shl(CONT, CONTq, 3);
    // OST at the first byte of the character that ends at byte i-1
    const uint64_t PLOST = shl(OST, OSTq, 1) | (shl(OST, OSTq, 2) & k1) | (shl(OST, OSTq, 3) & k1 & k2) |
                           (shl(OST, OSTq, 4) & k1 & k2 & k3);
    // letters: a match starts at a letter after CR/LF or a digit, after
    // punctuation unless that punctuation is one character that starts a
    // match (it then prefixes the letters), and inside a letter run only
    // where a contraction ended
    const uint64_t startL = L_ & LD & (SS | pCR | pN | (pO & ~PLOST) | (pL & R));
    const uint64_t startW_static = (Wst & ~pO) | (Wst & pO & ~CR_) | WL;
    o.static_starts = startL | OST | startW_static | SPST;
    o.K0 = o.K1 = o.K2 = o.K3 = o.todo = o.WstCR = 0;
  } else {
    const uint64_t APL = m.AP & LD;
    const uint64_t A1 = APL & ((s1 & nb1) | (ls & nb1 & nb2));
    const uint64_t A2 = APL & nb1 & nb2 & two & ~A1;
    const uint64_t SPm = SP_, WSm = NC & ~SP_;
    const uint64_t Um = m.LU & IN, Wm = m.LL & IN, Bm = m.LB & IN, Mm = m.M & IN;
    const uint64_t Om = O_ & ~Mm & ~A1 & ~A2;
    // kind codes: X0 CR1 SP2 WS3 N4 U5 W6 B7 M8 O9 A1=10 A2=11
    o.K0 = CR_ | WSm | Um | Bm | Om | A2;
    o.K1 = SPm | WSm | Wm | Bm | A1 | A2;
    o.K2 = N_ | Um | Wm | Bm;
    o.K3 = Mm | Om | A1 | A2;
    o.todo = m.lead & m.valid;  // special bytes are kind X
    o.WstCR = Wst & CR_;
    o.static_starts = (Wst & ~CR_) | WL | SPST;
  }

  // transfer functions
  uint32_t fd, fv;
  digit_v_fns(o, N_ & LD & (SS | ~pN), fd, fv);
  o.f_dig = fd;
  o.f_v = fv;
  if (G == 0) {
    uint32_t fc;
    if ((CR_ & ~SS) == ~uint64_t(0)) {
      fc = ((pO & 1) ? 1u : 2u) | (1u << 2) | (2u << 4);
    } else {
      uint64_t e2;
      fc = cr_runs(CR_, IN, SS, pO, NC & LD, 0u, e2) * 0x15u;
    }
    o.f_cr = fc;
    o.f_let = 0;
  } else {
    // the automaton over the word from every entry state; once all entry
    // states agree (after a space, a digit, a span start, ...) one state is
    // enough
    // (characters only, not every byte; and a kind whose step left the
    // function unchanged is skipped until the function changes again: runs
    // of letters and marks settle after a character or two)
    uint64_t f = FLET_ID;
    bool konst = false;
    uint32_t cst = 0;
    uint32_t settled = 0;  // kinds whose step is known to leave f unchanged
    for (uint64_t todo = o.todo; todo; todo &= todo - 1) {
      const int i = __ffsll(static_cast<unsigned long long>(todo)) - 1;
      const uint32_t k = uint32_t((o.K0 >> i) & 1) | (uint32_t((o.K1 >> i) & 1) << 1) |
                         (uint32_t((o.K2 >> i) & 1) << 2) | (uint32_t((o.K3 >> i) & 1) << 3);
      if ((SS >> i) & 1) {
        konst = true;
        cst = S_F;
      }
      if (!konst && ((settled >> k) & 1)) continue;
      uint64_t t;
      uint32_t sm;
      let_kind(k, t, sm);
      if (konst) {
        cst = flet_apply(t, cst);
      } else {
        const uint64_t g = flet_then(f, t);
        settled = g == f ? (settled | (1u << k)) : 0u;
        f = g;
        if ((f & 15u) * FLET_ONES == f) {
          konst = true;
          cst = uint32_t(f & 15u);
        }
      }
    }
    o.f_let = konst ? uint64_t(cst) * FLET_ONES : f;
    o.f_cr = 0;
  }
}

// 2-bit images (state s at bits 2s..2s+1) spread to one byte each
__device__ __forceinline__ uint32_t spread2(uint32_t f) {
  return (f & 3u) | ((f & 0xCu) << 6) | ((f & 0x30u) << 12) | ((f & 0xC0u) << 18);
}
template <int G>
__device__ __forceinline__ uint64_t pack_word_fn(const SplitWord &o) {
  if (G == 0)  // (the CR function's byte 3 is never selected: its states are 0..2)
    return fn_with_v<G>(uint64_t(spread2(o.f_dig)) | (uint64_t(spread2(o.f_cr)) << 32), o.f_v);
  return uint64_t(o.f_dig) | (uint64_t(o.f_v) << 8) | (o.f_let << 16);
}

// Per-byte machines with known inputs: digit-group starts, the v bits (VN
// bit i = v at byte i+1), and the CR machine (cl100k) or the letter
// automaton (o200k-style).  xs = CR state or automaton state entering the
// word.
template <int G>
__device__ __forceinline__ uint64_t split_finish(const SplitWord &o, uint64_t pCRmask, uint32_t ph,
                                                 uint32_t xs, uint32_t v, bool r50k) {
  uint64_t PH0 = 0, E2b = 0, VN = 0, extra = 0;
  const uint64_t NLD = o.N_ & o.LD;
  const uint64_t runstart = NLD & (o.SS | ~o.pN);
  if (r50k) {
    // one match per digit run; a U+0020 right before the run (in the same
    // span) is always a match start under the whitespace rules, and here
    // it leads the digits, so the run's own start goes
  } else if (o.N_ == NLD) {  // single-byte digits only
    PH0 = digit_phase0_ascii(NLD, runstart, ph);
  } else {
    for (int i = 0; i < 64; ++i) {
      const uint64_t b = bit(i);
      if (NLD & b) {
        ph = (runstart & b) ? 0u : (ph == 3u ? 0u : (ph + 1u) % 3u);
        if (ph == 0) PH0 |= b;
      } else if (!(o.N_ & b)) {
        ph = 3;
      }
    }
  }
  if (G == 0) {
    (void)cr_runs(o.CR_, o.IN, o.SS, o.pO, o.NC & o.LD, xs, E2b);
  } else {
    uint32_t st = xs;
    uint64_t LS = 0, PQ = 0, F1m = 0;
    for (uint64_t todo = o.todo; todo; todo &= todo - 1) {
      const int i = __ffsll(static_cast<unsigned long long>(todo)) - 1;
      const uint64_t b = bit(i);
      if (o.SS & b) st = S_F;
      const uint32_t k = uint32_t((o.K0 >> i) & 1) | (uint32_t((o.K1 >> i) & 1) << 1) |
                         (uint32_t((o.K2 >> i) & 1) << 2) | (uint32_t((o.K3 >> i) & 1) << 3);
      uint64_t t;
      uint32_t sm;
      let_kind(k, t, sm);
      PQ |= (st == S_Q || st == S_PS) ? b : 0;
      F1m |= (st == S_F1) ? b : 0;
      LS |= ((sm >> st) & 1) ? b : 0;
      st = flet_apply(t, st);
    }
    E2b = o.NC & o.LD & ~o.SS & F1m;
    extra = LS | (o.WstCR & ~PQ);
  }
  const uint64_t Qcand = o.NC & o.LD & pCRmask;
  if (Qcand) VN = v_next(o.BRK, o.NC, o.WS_, v);
  const uint64_t startN = r50k ? (runstart & ~o.pSP) : (NLD & (o.SS | ~o.pN | PH0));
  return o.static_starts | startN | E2b | extra | (Qcand & VN);
}

__device__ __forceinline__ void lane_setup(const EncodeArgs &a, int lane, uint32_t t, int64_t &w,
                                           WordMasks &m, Window &win) {
  w = int64_t(t) * TILE_WORDS + lane - 1;
  load_window(a.text, a.n, w * 64, win);
  uint64_t seg_lo, seg_hi;
  uint32_t seg_at;
  word_setup<false>(a, w, false, win, seg_lo, seg_hi, seg_at, m);
}

// previous-byte CR/LF within the span (needed by the emit pass)
__device__ __forceinline__ uint64_t prev_cr(const SplitWord &o) {
  const uint64_t q = shfl_up64(o.CR_, 1);
  return shl(o.CR_, q, 1) & ~o.SS;
}

// Wave scans of the lanes' packed functions: LTR parts inclusive in lane
// order, the v part inclusive in reverse lane order.
template <int G>
__device__ __forceinline__ void wave_scan_fns(uint64_t &ltr, uint32_t &fv, int lane) {
  ltr = wave_incl_scan(ltr, ltr_id<G>(), [](uint64_t x, uint64_t y) { return ltr_then<G>(x, y); });
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t nv = __shfl_down(fv, d, 64);
    if (lane + d < 64) fv = fv_then(nv, fv);
  }
}

// Step 4: per-tile transfer functions.
template <int G>
__device__ __forceinline__ void split_agg_body(const EncodeArgs &a) {
  const int lane = threadIdx.x;
  const uint32_t t = blockIdx.x;
  int64_t w;
  WordMasks m;
  Window win;
  lane_setup(a, lane, t, w, m, win);  // (its reads are bounded whatever the offsets)
  if (a.ws.status->pad2) return;      // checked once the word's loads are issued
  SplitWord o;
  split_word<G>(a, w, m, o);
  const bool owned = lane >= 1 && lane <= int(TILE_WORDS);
  const uint64_t pk = pack_word_fn<G>(o);
  uint64_t ltr = owned ? fn_ltr<G>(pk) : ltr_id<G>();
  uint32_t fv = owned ? o.f_v : FV_ID;
  wave_scan_fns<G>(ltr, fv, lane);
  const uint32_t fv0 = __shfl(fv, 0, 64);
  if (lane == 63) a.ws.tile_fn[t] = fn_with_v<G>(ltr, fv0);
}
__global__ void __launch_bounds__(64) k_split_agg(EncodeArgs a) { split_agg_body<0>(a); }
__global__ void __launch_bounds__(64) k_split_agg_o200k(EncodeArgs a) { let_fill(); split_agg_body<1>(a); }

// Step 5 (one workgroup): the carried state entering every tile.
template <int G>
__device__ __forceinline__ void scan_split_body(const EncodeArgs &a) {
  if (a.ws.status->pad2) return;
  __shared__ uint64_t s_f[1024];
  __shared__ uint32_t s_g[1024];
  const uint32_t T = a.n_tiles;
  const uint32_t tid = threadIdx.x;
  const uint32_t per = (T + 1023) / 1024;
  const uint32_t t0 = tid * per, t1 = min(T, t0 + per);
  uint64_t f = ltr_id<G>();
  uint32_t gv = FV_ID;
  // (each thread's tiles FOLD_BATCH at a time, a batch's loads issued first)
  fold_run(a.ws.tile_fn, t0, t1, [&](uint32_t, uint64_t x) { f = ltr_then<G>(f, fn_ltr<G>(x)); });
  fold_run_rev(a.ws.tile_fn, t0, t1, [&](uint32_t, uint64_t x) { gv = fv_then(gv, fn_v<G>(x)); });
  // scans over threads: LTR for (digit, CR / letter), RTL for v
  __shared__ uint64_t s_wf[33];
  __shared__ uint32_t s_wg[33];
  uint64_t all_f;
  const uint64_t in_f = block_incl_scan<1024>(
      f, ltr_id<G>(), [](uint64_t x, uint64_t y) { return ltr_then<G>(x, y); }, s_wf, all_f);
  const uint32_t in_g = block_incl_scan_rev<1024>(
      gv, FV_ID, [](uint32_t x, uint32_t y) { return fv_then(x, y); }, s_wg);
  // exclusive: the inclusive value of the neighbouring thread
  s_f[tid] = in_f;
  s_g[tid] = in_g;
  __syncthreads();
  const uint64_t ex_f = tid > 0 ? s_f[tid - 1] : ltr_id<G>();
  const uint32_t ex_g = tid + 1 < 1024 ? s_g[tid + 1] : FV_ID;
  // the text starts outside any digit run, with no CR run / in state F
  uint32_t dig = ltr_apply_dig<G>(ex_f, 3u);
  uint32_t x = ltr_apply_x<G>(ex_f, 0u);
  uint32_t v = fv_apply(ex_g, 0u);  // past the end of the text: a break
  // the state entering every tile: the left-to-right parts forward, the
  // lookahead backward, each tile's carry written once
  for (uint32_t q = t0; q < t1; q += FOLD_BATCH) {
    uint64_t fn[FOLD_BATCH];
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) fn[j] = q + j < t1 ? a.ws.tile_fn[q + j] : 0ull;
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
      if (q + j >= t1) continue;
      a.ws.tile_carry[q + j] = dig | (x << 8);  // (the lookahead is added below)
      dig = ltr_apply_dig<G>(fn[j], dig);
      x = ltr_apply_x<G>(fn[j], x);
    }
  }
  for (uint32_t q = t1; q > t0; q -= min(q - t0, FOLD_BATCH)) {
    uint64_t fn[FOLD_BATCH];
    uint32_t cv[FOLD_BATCH];
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
      const bool in = q - t0 > j;
      fn[j] = in ? a.ws.tile_fn[q - 1 - j] : 0ull;
      cv[j] = in ? a.ws.tile_carry[q - 1 - j] : 0u;
    }
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
      if (q - t0 <= j) continue;
      a.ws.tile_carry[q - 1 - j] = (cv[j] & 0xFFFFu) | (v << 16);
      v = fv_apply(fn_v<G>(fn[j]), v);
    }
  }
}
__global__ void __launch_bounds__(1024) k_scan_split(EncodeArgs a) { scan_split_body<0>(a); }
__global__ void __launch_bounds__(1024) k_scan_split_o200k(EncodeArgs a) { scan_split_body<1>(a); }

// The state entering tile t, folded from the tile functions directly (for
// texts of at most FUSE_TILES tiles, in place of the tile scan): the
// left-to-right parts over tiles [0, t) from the text start (outside any
// digit run, no CR run / state F), the lookahead over tiles (t, T) from past
// the text end (a break).  Lane l folds a contiguous run of tiles; the runs
// compose in lane order by wave shuffles.  Must be called by all 64 lanes.
template <int G>
__device__ __forceinline__ uint32_t carry_direct(const EncodeArgs &a, uint32_t t, int lane) {
  const uint32_t T = a.n_tiles;
  const uint32_t per_l = (t + 63) / 64, per_r = (T - 1 - t + 63) / 64;
  uint64_t f = ltr_id<G>();
  const uint32_t l0 = min(t, uint32_t(lane) * per_l), l1 = min(t, l0 + per_l);
  fold_run(a.ws.tile_fn, l0, l1, [&](uint32_t, uint64_t x) { f = ltr_then<G>(f, fn_ltr<G>(x)); });
  uint32_t gv = FV_ID;
  const uint32_t r0 = min(T, t + 1 + uint32_t(lane) * per_r), r1 = min(T, r0 + per_r);
  fold_run_rev(a.ws.tile_fn, r0, r1, [&](uint32_t, uint64_t x) { gv = fv_then(gv, fn_v<G>(x)); });
  wave_scan_fns<G>(f, gv, lane);
  const uint64_t all_f = __shfl(static_cast<unsigned long long>(f), 63, 64);
  const uint32_t all_g = __shfl(gv, 0, 64);
  const uint32_t dig = ltr_apply_dig<G>(all_f, 3u);
  const uint32_t x = ltr_apply_x<G>(all_f, 0u);
  const uint32_t v = fv_apply(all_g, 0u);
  return dig | (x << 8) | (v << 16);
}

// Entries of the list of merge-unit positions that a wave checks at once.
constexpr uint32_t REST_LIST = 1024;

// Merge-unit cuts among K positions j (stage indexes, >= 16, of the wave's
// staged bytes b32), for positions whose byte pair occurs inside a key: j is
// a cut when neither 3-byte window across it is a key, the pair itself is
// not one, and no 4-byte window across it may occur inside a key.  Bit k of
// the result: position k (with has[k]) is a cut.  The table loads of all K
// positions are issued together.
template <int K>
__device__ __forceinline__ uint32_t unit_cuts(const DevTables &T, const uint32_t *b32, const uint32_t *pos,
                                              const bool *has) {
  uint32_t hit[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    // bytes j-3 .. j+4
    const uint32_t q = pos[k] - 3u, d = q >> 2, sh = q & 3u;
    const uint32_t x0 = b32[d], x1 = b32[d + 1], x2 = b32[d + 2];
    const uint32_t lo4 = __builtin_amdgcn_alignbyte(x1, x0, sh);
    const uint32_t hi4 = __builtin_amdgcn_alignbyte(x2, x1, sh);
    const uint32_t v0 = lo4;                                      // j-3 .. j
    const uint32_t v1 = __builtin_amdgcn_alignbyte(hi4, lo4, 1);  // j-2 .. j+1
    const uint32_t v2 = __builtin_amdgcn_alignbyte(hi4, lo4, 2);  // j-1 .. j+2
    const uint32_t x3a = __builtin_bswap32(v1) >> 8;  // bytes j-2, j-1, j, first byte high
    const uint32_t x3b = __builtin_bswap32(v2) >> 8;  // bytes j-1, j, j+1
    const uint32_t pr = ((v2 & 0xFFu) << 8) | ((v2 >> 8) & 0xFFu);  // bytes j-1, j
    const uint32_t q0 = q4_index(v0), q1 = q4_index(v1), q2 = q4_index(v2);
    const bool pk = T.pair[pr] != RANK_NONE;
    const uint32_t h = ((T.k3[x3a >> 5] >> (x3a & 31)) | (T.k3[x3b >> 5] >> (x3b & 31)) |
                        (T.q4[q0 >> 5] >> (q0 & 31)) | (T.q4[q1 >> 5] >> (q1 & 31)) |
                        (T.q4[q2 >> 5] >> (q2 & 31))) & 1u;
    hit[k] = h | (pk ? 1u : 0u);
  }
  uint32_t cuts = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) cuts |= (has[k] && !hit[k]) ? (1u << k) : 0u;
  return cuts;
}

// Step 6: piece-start bits of every word and the number of pieces per tile.
template <int G>
__device__ __forceinline__ void split_body(const EncodeArgs &a) {
  const int lane = threadIdx.x;
  const uint32_t t = blockIdx.x;
  int64_t w;
  WordMasks m;
  Window win;
  lane_setup(a, lane, t, w, m, win);  // (its reads are bounded whatever the offsets)
  if (a.ws.status->pad2) return;      // checked once the word's loads are issued
  SplitWord o;
  split_word<G>(a, w, m, o);
  const bool owned = lane >= 1 && lane <= int(TILE_WORDS) && w < int64_t(a.n_words);
  const bool mine = lane >= 1 && lane <= int(TILE_WORDS);
  const uint64_t pk = pack_word_fn<G>(o);
  uint64_t ltr = mine ? fn_ltr<G>(pk) : ltr_id<G>();
  uint32_t fv = mine ? o.f_v : FV_ID;
  wave_scan_fns<G>(ltr, fv, lane);
  // exclusive: state entering this lane's word
  uint64_t exl = __shfl_up(static_cast<unsigned long long>(ltr), 1, 64);
  uint32_t exv = __shfl_down(fv, 1, 64);
  if (lane == 0) exl = ltr_id<G>();
  if (lane == 63) exv = FV_ID;
  const uint32_t carry = a.n_tiles <= FUSE_TILES ? carry_direct<G>(a, t, lane) : a.ws.tile_carry[t];
  const uint32_t ph = ltr_apply_dig<G>(exl, carry & 0xFFu);
  const uint32_t xs = ltr_apply_x<G>(exl, (carry >> 8) & 0xFFu);
  const uint32_t v = fv_apply(exv, (carry >> 16) & 1u);
  const uint64_t pCRm = prev_cr(o);
  const bool r50k = G == 0 && a.T.grammar == BBPE_GRAMMAR_R50K_STYLE;
  uint64_t ps = split_finish<G>(o, pCRm, ph, xs, v, r50k) & m.valid;
  if (a.merge_units) {
    // Merge units: where no key can occur across a position, no merge ever
    // crosses it (every part is a key), so the piece is cut there into
    // independent units.  A key occurrence across position j (between bytes
    // j-1 and j) contains the byte pair there; if it is 2 or 3 bytes long it
    // is one of the windows [j-1, j+1), [j-2, j+1), [j-1, j+2); if longer, it
    // contains one of the 4-byte windows starting at j-3, j-2, j-1.  So j is
    // a cut when the pair occurs inside no key, or else when neither short
    // window is a key and no 4-byte window occurs inside a key (windows that
    // reach outside the piece only make the test stricter).  Checked where a
    // non-ASCII byte is involved and where a lower-case letter is followed by
    // an upper-case one (identifiers in code), which is where long pieces
    // come from; skipping a check only leaves a unit longer, never changes
    // the ids.
    // The pair bitmap goes to LDS first (8 KB, only in waves that have a
    // candidate), and every position is checked without a branch, so that
    // the reads overlap.
    __shared__ __align__(16) uint32_t s_inner[2048];
    __shared__ uint4 s_bytes[STAGE_BYTES / 16];
    const uint64_t na_prev = shfl_up64(m.na, 1), ll_prev = shfl_up64(m.LL, 1);
    const uint64_t cand = o.IN & ~ps & ~o.SS & m.valid &
                          (m.na | shl(m.na, na_prev, 1) | (m.LU & shl(m.LL, ll_prev, 1)));
    if (__ballot(cand != 0)) {
      const uint4 *src = reinterpret_cast<const uint4 *>(a.T.inner);
      uint4 *dst = reinterpret_cast<uint4 *>(s_inner);
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[k * 64 + lane] = src[k * 64 + lane];
      stage_window(s_bytes, win, lane);
      __syncthreads();
      uint64_t cut = 0;
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const uint32_t pr = (win.at(i - 1) << 8) | win.at(i);
        cut |= uint64_t(((s_inner[pr >> 5] >> (pr & 31)) & 1) ^ 1u) << i;
      }
      ps |= cand & cut;
      // pairs that occur inside keys: the longer windows, at character
      // boundaries only, eight positions at a time with their loads issued
      // together.  Where one lane has many more positions than the wave's
      // average (so more rounds of loads), the wave's positions go to a
      // list shared out over its lanes (every 64th entry each) and a cut
      // found goes back to its word in LDS; else each lane takes its own.
      const uint64_t rest = owned ? (cand & ~cut & m.lead) : 0ull;
      const uint32_t cnt = uint32_t(__popcll(rest));
      const uint32_t incl = wave_incl_sum(cnt, lane);
      const uint32_t total = __shfl(incl, 63, 64);
      uint32_t most = cnt;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) most = max(most, uint32_t(__shfl_xor(most, d, 64)));
      const uint32_t *b32 = reinterpret_cast<const uint32_t *>(s_bytes);
      if ((most + 7) / 8 > (total + 511) / 512) {  // (wave-uniform)
        // the list and the cuts take the pair bitmap's place
        static_assert(REST_LIST * 2 + 64 * 8 <= sizeof(s_inner), "list space");
        uint16_t *s_list = reinterpret_cast<uint16_t *>(s_inner);
        unsigned long long *s_cut = reinterpret_cast<unsigned long long *>(s_inner + REST_LIST / 2);
        __syncthreads();
        s_cut[lane] = 0;
        const uint32_t w0 = 16u + 64u * uint32_t(lane);  // the word's first byte in the stage
        for (uint32_t c0 = 0; c0 < total; c0 += REST_LIST) {
          const uint32_t c1 = min(total, c0 + REST_LIST);
          uint32_t k = incl - cnt;
          for (uint64_t x = rest; x && k < c1; x &= x - 1, ++k)
            if (k >= c0) s_list[k - c0] = uint16_t(w0 + uint32_t(__ffsll(static_cast<unsigned long long>(x)) - 1));
          __syncthreads();
          for (uint32_t g0 = 0; g0 < c1 - c0; g0 += 64u * 8u) {
            constexpr int K = 8;
            uint32_t pos[K];
            bool has[K];
#pragma unroll
            for (int k2 = 0; k2 < K; ++k2) {
              const uint32_t g = g0 + uint32_t(lane) + 64u * uint32_t(k2);
              has[k2] = g < c1 - c0;
              pos[k2] = s_list[has[k2] ? g : 0u];
            }
            const uint32_t cuts = unit_cuts<K>(a.T, b32, pos, has);
#pragma unroll
            for (int k2 = 0; k2 < K; ++k2)
              if ((cuts >> k2) & 1u) atomicOr(&s_cut[(pos[k2] - 16u) >> 6], 1ull << ((pos[k2] - 16u) & 63u));
          }
          __syncthreads();
        }
        ps |= s_cut[lane];
      } else {
        const uint32_t w0 = 16u + 64u * uint32_t(lane);
        for (uint64_t x = rest; x;) {
          constexpr int K = 8;
          uint32_t pos[K];
          bool has[K];
          int ii[K];
#pragma unroll
          for (int k2 = 0; k2 < K; ++k2) {
            ii[k2] = __ffsll(static_cast<unsigned long long>(x)) - 1;  // -1 once none are left
            x &= x - 1;
            has[k2] = ii[k2] >= 0;
            pos[k2] = w0 + uint32_t(has[k2] ? ii[k2] : 0);
          }
          const uint32_t cuts = unit_cuts<K>(a.T, b32, pos, has);
#pragma unroll
          for (int k2 = 0; k2 < K; ++k2)
            if ((cuts >> k2) & 1u) ps |= bit(ii[k2]);
        }
      }
    }
  }
  const uint32_t np = owned ? uint32_t(__popcll(ps)) : 0u;
  if (owned) a.ws.ps[w] = ps;
  const uint32_t tot = wave_sum(np);
  if (lane == 0) a.ws.tile_np[t] = tot;
}
__global__ void __launch_bounds__(64) k_split(EncodeArgs a) { split_body<0>(a); }
__global__ void __launch_bounds__(64) k_split_o200k(EncodeArgs a) { let_fill(); split_body<1>(a); }

}  // namespace bbpe
