// Split of every span into pre-tokens (cl100k grammar), as piece-start bits.
//
// The printed pattern is applied leftmost-first with possessive quantifiers
// (tiktoken deep-dive page, "The split pattern").  Rather than running a
// regex engine, each lane derives the match starts of its 64-byte word from
// class bitmasks: whether a match starts at a character depends only on the
// characters a few bytes around it, except for three quantities that are
// carried along the text:
//   * the position of a digit inside its digit run, modulo 3 (digit groups of
//     at most three);
//   * whether a run of CR/LF characters at the start of a whitespace run was
//     preceded by punctuation (the punctuation clause then swallows those
//     CR/LF characters, and the whitespace clauses restart after them);
//   * whether a run of non-CR/LF whitespace reaches a non-space character of
//     the same span (the last CR/LF of a whitespace run ends a match only if
//     the whitespace after it is followed by a non-space character).
// The first two flow left to right, the third right to left.  Each lane
// summarises its word as a transfer function on the carried state; functions
// compose across lanes (wave scans) and across tiles (a one-workgroup scan).
#include <hip/hip_runtime.h>

#include "bbpe_classify.h"
#include "bbpe_device.h"
#include "bbpe_kernels.h"

namespace bbpe {

// Transfer-function encodings.
//   digit phase: states 0,1,2 (index of the last digit in its run, mod 3) and
//                3 (not in a digit run); 4 entries of 2 bits.
//   CR run:      states 0 (none), 1 (CR/LF run that followed punctuation),
//                2 (other CR/LF run); 3 entries of 2 bits.
//   v (RTL):     state = "the non-CR/LF whitespace continuing here ends at a
//                non-space character of the span"; 2 entries of 1 bit.
constexpr uint32_t FDIG_ID = 0xE4u;  // 3,2,1,0
constexpr uint32_t FCR_ID = 0x24u;   // 2,1,0
constexpr uint32_t FV_ID = 0x2u;     // 1,0

__device__ __forceinline__ uint32_t fdig_apply(uint32_t f, uint32_t s) { return (f >> (2 * s)) & 3u; }
__device__ __forceinline__ uint32_t fcr_apply(uint32_t f, uint32_t s) { return (f >> (2 * s)) & 3u; }
__device__ __forceinline__ uint32_t fv_apply(uint32_t f, uint32_t s) { return (f >> s) & 1u; }
// f first, then g
__device__ __forceinline__ uint32_t fdig_then(uint32_t f, uint32_t g) {
  uint32_t h = 0;
#pragma unroll
  for (uint32_t s = 0; s < 4; ++s) h |= fdig_apply(g, fdig_apply(f, s)) << (2 * s);
  return h;
}
__device__ __forceinline__ uint32_t fcr_then(uint32_t f, uint32_t g) {
  uint32_t h = 0;
#pragma unroll
  for (uint32_t s = 0; s < 3; ++s) h |= fcr_apply(g, fcr_apply(f, s)) << (2 * s);
  return h;
}
__device__ __forceinline__ uint32_t fv_then(uint32_t f, uint32_t g) {
  uint32_t h = 0;
#pragma unroll
  for (uint32_t s = 0; s < 2; ++s) h |= fv_apply(g, fv_apply(f, s)) << s;
  return h;
}
// packed: bits 0-7 digit, 8-13 CR, 16-17 v
__device__ __forceinline__ uint32_t pack_fn(uint32_t d, uint32_t c, uint32_t v) {
  return d | (c << 8) | (v << 16);
}

struct SplitWord {
  // carried-state inputs to the per-byte machines
  uint64_t SS, SPST, IN, BRK, LD, N_, CR_, NC, WS_, pN, pO;
  uint64_t static_starts;  // starts that need no carried state
  uint32_t f_dig, f_cr, f_v;
};

// Everything of the split that does not depend on the carried states, plus
// this word's transfer functions.  Must be called by all 64 lanes.
__device__ __forceinline__ void split_word_g1(const EncodeArgs &a, int64_t w, const WordMasks &m,
                                              SplitWord &o) {
  const bool inrange = w >= 0 && w < int64_t(a.n_words);
  const uint64_t SS = inrange ? a.ws.ss[w] : 0;
  const uint64_t SPST = inrange ? a.ws.spst[w] : 0;
  const uint64_t SPC = inrange ? a.ws.spc[w] : 0;
  const uint64_t IN = m.valid & ~SPC;
  const uint64_t BRK = SS | SPST | ~m.valid;
  const uint64_t L_ = m.L & IN, N_ = m.N & IN, WS_ = m.WS & IN, CR_ = m.CR & IN, SP_ = m.SP & IN;
  const uint64_t O_ = IN & ~(m.L | m.N | m.WS);
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

  // punctuation (any non-letter, non-digit, non-space character): a match
  // starts at the first character of a punctuation run unless a single
  // space before it joins the run
  const uint64_t OST = O_ & LD & ~pO & ~pSP;
  // an apostrophe that starts a match and is followed, inside the span, by
  // s d m t (either case, or U+017F) or ll / ve / re: the contraction clause
  const uint64_t APc = m.AP & OST;
  const uint64_t nb1 = shr(INB, INBn, 1), nb2 = shr(INB, INBn, 2);
  const uint64_t s1 = shr(m.c_sdmt, sdmtn, 1);
  const uint64_t C2M = APc & s1 & nb1;  // the match ends two bytes on
  const uint64_t ls = shr(m.c_ls0, ls0n, 1) & shr(m.c_ls1, ls1n, 2);
  const uint64_t two = (shr(m.c_l, ln, 1) & shr(m.c_l, ln, 2)) | (shr(m.c_v, vn, 1) & shr(m.c_e, en, 2)) |
                       (shr(m.c_r, rn, 1) & shr(m.c_e, en, 2));
  const uint64_t C3M = APc & nb1 & nb2 & (ls | (two & ~s1));  // three bytes on

  const uint64_t OSTq = shfl_up64(OST, 1), C2q = shfl_up64(C2M, 1), C3q = shfl_up64(C3M, 1);
  const uint64_t R = shl(C2M, C2q, 2) | shl(C3M, C3q, 3);
  const uint64_t k1 = shl(CONT, CONTq, 1), k2 = shl(CONT, CONTq, 2), k3 = shl(CONT, CONTq, 3);
  // OST at the first byte of the character that ends at byte i-1
  const uint64_t PLOST = shl(OST, OSTq, 1) | (shl(OST, OSTq, 2) & k1) | (shl(OST, OSTq, 3) & k1 & k2) |
                         (shl(OST, OSTq, 4) & k1 & k2 & k3);
  // letters: a match starts at a letter after CR/LF or a digit, after
  // punctuation unless that punctuation is one character that starts a match
  // (it then prefixes the letters), and inside a letter run only where a
  // contraction ended
  const uint64_t startL = L_ & LD & (SS | pCR | pN | (pO & ~PLOST) | (pL & R));

  // whitespace: a run starts a match where it begins, unless punctuation
  // before it swallowed its leading CR/LF characters (handled by the CR
  // machine); the last non-CR/LF character of a run starts a match when a
  // non-space character of the span follows; the first character after the
  // run's last CR/LF starts one when the rest of the run is followed by a
  // non-space character (the v machine)
  const uint64_t Wst = WS_ & LD & ~pWS;
  const uint64_t NC = WS_ & ~CR_;
  const uint64_t n1 = shr(GL, GLn, 1), kn1 = shr(CONT, CONTn, 1), kn2 = shr(CONT, CONTn, 2);
  const uint64_t kn3 = shr(CONT, CONTn, 3);
  const uint64_t nextGL = n1 | (shr(GL, GLn, 2) & kn1) | (shr(GL, GLn, 3) & kn1 & kn2) |
                          (shr(GL, GLn, 4) & kn1 & kn2 & kn3);
  const uint64_t WL = NC & LD & nextGL;
  const uint64_t startW_static = (Wst & ~pO) | (Wst & pO & ~CR_) | WL;

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
  o.static_starts = startL | OST | startW_static | SPST;

  // transfer functions
  // digits: identity-like (shift by count) only when the whole word continues a digit run
  {
    const uint64_t runstart = N_ & LD & (SS | ~pN);
    uint32_t fd;
    if (N_ == ~uint64_t(0) && runstart == 0) {
      const uint32_t cnt = uint32_t(__popcll(LD)) % 3u;
      fd = 0;
#pragma unroll
      for (uint32_t s = 0; s < 3; ++s) fd |= ((s + cnt) % 3u) << (2 * s);
      fd |= ((cnt + 2u) % 3u) << 6;
    } else {
      uint32_t ph = 3;
      for (int i = 0; i < 64; ++i) {
        const uint64_t b = bit(i);
        if (N_ & LD & b) ph = (runstart & b) ? 0u : (ph == 3u ? 0u : (ph + 1u) % 3u);
        else if (!(N_ & b)) ph = 3;
      }
      fd = ph * 0x55u;  // constant function
    }
    o.f_dig = fd;
  }
  {
    uint32_t fc;
    if ((CR_ & ~SS) == ~uint64_t(0)) {
      fc = ((pO & 1) ? 1u : 2u) | (1u << 2) | (2u << 4);
    } else {
      uint32_t st = 0;
      for (int i = 0; i < 64; ++i) {
        const uint64_t b = bit(i);
        if (!(IN & b)) st = 0;
        else if (CR_ & b) st = (SS & b) ? 2u : (st == 0 ? ((pO & b) ? 1u : 2u) : st);
        else st = 0;
      }
      fc = st * 0x15u;
    }
    o.f_cr = fc;
  }
  {
    const uint64_t prop = NC & ~BRK;
    uint32_t fv;
    if (prop == ~uint64_t(0)) {
      fv = FV_ID;
    } else {
      // v at byte 0 is fixed by the first non-propagating byte
      const int i = __ffsll(static_cast<unsigned long long>(~prop)) - 1;
      const uint64_t b = bit(i);
      const uint32_t v = (BRK & b) ? 0u : ((WS_ & b) ? 0u : 1u);
      fv = v * 3u;
    }
    o.f_v = fv;
  }
}

// Per-byte machines with known inputs: digit-group starts, the whitespace
// restart after swallowed CR/LF, and the v bits (VN bit i = v at byte i+1).
__device__ __forceinline__ uint64_t split_finish_g1(const SplitWord &o, uint64_t pCRmask, uint32_t ph,
                                                    uint32_t st, uint32_t v) {
  uint64_t PH0 = 0, E2b = 0, VN = 0;
  const uint64_t NLD = o.N_ & o.LD;
  const uint64_t runstart = NLD & (o.SS | ~o.pN);
  if (o.N_) {
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
  if (o.CR_ | (st != 0)) {
    for (int i = 0; i < 64; ++i) {
      const uint64_t b = bit(i);
      if (!(o.IN & b)) {
        st = 0;
      } else if (o.CR_ & b) {
        st = (o.SS & b) ? 2u : (st == 0 ? ((o.pO & b) ? 1u : 2u) : st);
      } else {
        if (st == 1 && (o.NC & o.LD & b) && !(o.SS & b)) E2b |= b;
        st = 0;
      }
    }
  }
  const uint64_t Qcand = o.NC & o.LD & pCRmask;
  if (Qcand) {
    for (int i = 63; i >= 0; --i) {
      const uint64_t b = bit(i);
      if (v) VN |= b;
      if (o.BRK & b) v = 0;
      else if (o.NC & b) { /* propagate */ }
      else v = (o.WS_ & b) ? 0u : 1u;
    }
  }
  const uint64_t startN = NLD & (o.SS | ~o.pN | PH0);
  return o.static_starts | startN | E2b | (Qcand & VN);
}

__device__ __forceinline__ void lane_setup(const EncodeArgs &a, int lane, uint32_t t, int64_t &w,
                                           WordMasks &m, Window &win) {
  w = int64_t(t) * TILE_WORDS + lane - 1;
  const int64_t base = w * 64;
  load_window(a.text, a.n, base, win);
  uint64_t seg_lo, seg_hi;
  uint32_t seg_at;
  segment_marks(a.seg_off, a.n_seg, base, seg_lo, seg_hi, seg_at);
  classify_word(a.T, a.text, win, base, a.n, seg_lo, seg_hi, m);
}

// previous-byte CR/LF within the span (needed by the emit pass)
__device__ __forceinline__ uint64_t prev_cr(const SplitWord &o) {
  const uint64_t q = shfl_up64(o.CR_, 1);
  return shl(o.CR_, q, 1) & ~o.SS;
}

// Step 4: per-tile transfer functions.
__global__ void __launch_bounds__(64) k_split_agg(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  const int lane = threadIdx.x;
  const uint32_t t = blockIdx.x;
  int64_t w;
  WordMasks m;
  Window win;
  lane_setup(a, lane, t, w, m, win);
  SplitWord o;
  split_word_g1(a, w, m, o);
  const bool owned = lane >= 1 && lane <= int(TILE_WORDS);
  uint32_t fd = owned ? o.f_dig : FDIG_ID, fc = owned ? o.f_cr : FCR_ID, fv = owned ? o.f_v : FV_ID;
  // left-to-right composition (lane order) and right-to-left for v
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t pd = __shfl_up(fd, d, 64), pc = __shfl_up(fc, d, 64);
    const uint32_t nv = __shfl_down(fv, d, 64);
    if (lane >= d) {
      fd = fdig_then(pd, fd);
      fc = fcr_then(pc, fc);
    }
    if (lane + d < 64) fv = fv_then(nv, fv);
  }
  const uint32_t fv0 = __shfl(fv, 0, 64);
  if (lane == 63) a.ws.tile_fn[t] = pack_fn(fd, fc, fv0);
}

// Step 5 (one workgroup): the carried state entering every tile.
__global__ void __launch_bounds__(1024) k_scan_split(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  __shared__ uint32_t s_f[1024];
  __shared__ uint32_t s_g[1024];
  const uint32_t T = a.n_tiles;
  const uint32_t tid = threadIdx.x;
  const uint32_t per = (T + 1023) / 1024;
  const uint32_t t0 = tid * per, t1 = min(T, t0 + per);
  uint32_t fd = FDIG_ID, fc = FCR_ID, gv = FV_ID;
  for (uint32_t t = t0; t < t1; ++t) {
    const uint32_t f = a.ws.tile_fn[t];
    fd = fdig_then(fd, f & 0xFFu);
    fc = fcr_then(fc, (f >> 8) & 0x3Fu);
  }
  for (uint32_t t = t1; t > t0; --t) gv = fv_then(gv, (a.ws.tile_fn[t - 1] >> 16) & 3u);
  s_f[tid] = fd | (fc << 8);
  s_g[tid] = gv;
  __syncthreads();
  // exclusive scans over threads: LTR for (digit, CR), RTL for v
  for (uint32_t d = 1; d < 1024; d <<= 1) {
    const uint32_t lf = tid >= d ? s_f[tid - d] : (FDIG_ID | (FCR_ID << 8));
    const uint32_t rg = tid + d < 1024 ? s_g[tid + d] : FV_ID;
    __syncthreads();
    const uint32_t cur = s_f[tid];
    s_f[tid] = fdig_then(lf & 0xFFu, cur & 0xFFu) | (fcr_then((lf >> 8) & 0x3Fu, (cur >> 8) & 0x3Fu) << 8);
    s_g[tid] = fv_then(rg, s_g[tid]);
    __syncthreads();
  }
  const uint32_t ex_f = tid > 0 ? s_f[tid - 1] : (FDIG_ID | (FCR_ID << 8));
  const uint32_t ex_g = tid + 1 < 1024 ? s_g[tid + 1] : FV_ID;
  uint32_t dig = fdig_apply(ex_f & 0xFFu, 3u);  // text starts outside any digit run
  uint32_t cr = fcr_apply((ex_f >> 8) & 0x3Fu, 0u);
  for (uint32_t t = t0; t < t1; ++t) {
    a.ws.tile_carry[t] = (a.ws.tile_carry[t] & ~0xFFFFu) | dig | (cr << 8);
    const uint32_t f = a.ws.tile_fn[t];
    dig = fdig_apply(f & 0xFFu, dig);
    cr = fcr_apply((f >> 8) & 0x3Fu, cr);
  }
  __syncthreads();
  uint32_t v = fv_apply(ex_g, 0u);  // past the end of the text: a break
  for (uint32_t t = t1; t > t0; --t) {
    a.ws.tile_carry[t - 1] = (a.ws.tile_carry[t - 1] & 0xFFFFu) | (v << 16);
    v = fv_apply((a.ws.tile_fn[t - 1] >> 16) & 3u, v);
  }
}

// Step 6: piece-start bits of every word and the number of pieces per tile.
__global__ void __launch_bounds__(64) k_split(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  const int lane = threadIdx.x;
  const uint32_t t = blockIdx.x;
  int64_t w;
  WordMasks m;
  Window win;
  lane_setup(a, lane, t, w, m, win);
  SplitWord o;
  split_word_g1(a, w, m, o);
  const bool owned = lane >= 1 && lane <= int(TILE_WORDS) && w < int64_t(a.n_words);
  uint32_t fd = (lane >= 1 && lane <= int(TILE_WORDS)) ? o.f_dig : FDIG_ID;
  uint32_t fc = (lane >= 1 && lane <= int(TILE_WORDS)) ? o.f_cr : FCR_ID;
  uint32_t fv = (lane >= 1 && lane <= int(TILE_WORDS)) ? o.f_v : FV_ID;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t pd = __shfl_up(fd, d, 64), pc = __shfl_up(fc, d, 64);
    const uint32_t nv = __shfl_down(fv, d, 64);
    if (lane >= d) {
      fd = fdig_then(pd, fd);
      fc = fcr_then(pc, fc);
    }
    if (lane + d < 64) fv = fv_then(nv, fv);
  }
  // exclusive: state entering this lane's word
  uint32_t exd = __shfl_up(fd, 1, 64), exc = __shfl_up(fc, 1, 64), exv = __shfl_down(fv, 1, 64);
  if (lane == 0) { exd = FDIG_ID; exc = FCR_ID; }
  if (lane == 63) exv = FV_ID;
  const uint32_t carry = a.ws.tile_carry[t];
  const uint32_t ph = fdig_apply(exd, carry & 0xFFu);
  const uint32_t st = fcr_apply(exc, (carry >> 8) & 0xFFu);
  const uint32_t v = fv_apply(exv, (carry >> 16) & 1u);
  const uint64_t pCRm = prev_cr(o);
  uint64_t ps = split_finish_g1(o, pCRm, ph, st, v) & m.valid;
  if (a.merge_units) {
    // Merge units: a byte pair that occurs inside no key can never be merged
    // across (the merged part would be a key containing it), so the piece is
    // cut there into independent units.  Checked where a non-ASCII byte is
    // involved, which is where long pieces come from; skipping a check only
    // leaves a unit longer, never changes the ids.
    const uint64_t na_prev = shfl_up64(m.na, 1);
    const uint64_t cand = o.IN & ~ps & ~o.SS & m.valid & (m.na | shl(m.na, na_prev, 1));
    if (cand) {
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        if ((cand >> i) & 1) {
          const uint32_t pr = (win.at(i - 1) << 8) | win.at(i);
          if (!((a.T.inner[pr >> 5] >> (pr & 31)) & 1)) ps |= bit(i);
        }
      }
    }
  }
  const uint32_t np = owned ? uint32_t(__popcll(ps)) : 0u;
  if (owned) a.ws.ps[w] = ps;
  const uint32_t tot = wave_sum(np);
  if (lane == 0) a.ws.tile_np[t] = tot;
}

}  // namespace bbpe
