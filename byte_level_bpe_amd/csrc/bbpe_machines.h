// Bit-parallel forms of the per-byte state machines of the split, over the
// 64 bytes of one word (bit i = byte i).  Each replaces a 64-step loop over
// the bytes with log-step segmented fills (shift, mask, or), whose result is
// the same for every input.
#pragma once

#include <stdint.h>

#include "bbpe_internal.h"

namespace bbpe {

BBPE_HD int hibit64(uint64_t x) { return x ? 63 - __builtin_clzll(x) : -1; }
// bits strictly above position x (x in [-1, 63])
BBPE_HD uint64_t above64(int x) { return x >= 63 ? 0ull : (~0ull << (x + 1)); }

// Positions reachable from the seeds S by steps i-1 -> i into positions of P.
BBPE_HD uint64_t fill_up(uint64_t S, uint64_t P) {
  S |= (S << 1) & P;  P &= P << 1;
  S |= (S << 2) & P;  P &= P << 2;
  S |= (S << 4) & P;  P &= P << 4;
  S |= (S << 8) & P;  P &= P << 8;
  S |= (S << 16) & P; P &= P << 16;
  S |= (S << 32) & P;
  return S;
}
// Positions reachable from S by steps i+1 -> i into positions of P.
BBPE_HD uint64_t fill_down(uint64_t S, uint64_t P) {
  S |= (S >> 1) & P;  P &= P >> 1;
  S |= (S >> 2) & P;  P &= P >> 2;
  S |= (S >> 4) & P;  P &= P >> 4;
  S |= (S >> 8) & P;  P &= P >> 8;
  S |= (S >> 16) & P; P &= P >> 16;
  S |= (S >> 32) & P;
  return S;
}

// Digit groups of at most three.  DL: digit characters' first bytes; RS:
// those that start a digit run; ph_in: the phase (0, 1, 2) of the last digit
// before the word, or 3 outside a run.  Returns the digits of phase 0 (each
// starts a match).  Valid when every digit byte is a first byte (single-byte
// digits), which makes each run a contiguous block of bits.
BBPE_HD uint64_t digit_phase0_ascii(uint64_t DL, uint64_t RS, uint32_t ph_in) {
  const uint64_t C = DL & ~RS;  // digits that continue a run
  uint64_t S = RS;
  if (C & 1) {  // the run entering the word: its first digit has phase p0
    const uint32_t p0 = ph_in == 3 ? 0u : (ph_in + 1) % 3;
    const uint32_t z = (3 - p0) % 3;  // first position of phase 0
    const uint64_t run = ~C ? ((1ull << __builtin_ctzll(~C)) - 1) : ~0ull;
    if ((run >> z) & 1) S |= 1ull << z;
  }
  // steps of three positions inside a run: i - 3 -> i when i-2, i-1, i
  // continue the run
  uint64_t P = C & (C << 1) & (C << 2);
  S |= (S << 3) & P;  P &= P << 3;
  S |= (S << 6) & P;  P &= P << 6;
  S |= (S << 12) & P; P &= P << 12;
  S |= (S << 24) & P; P &= P << 24;
  S |= (S << 48) & P;
  return S;
}

// Phase after the word when the word holds a reset (a byte that is no digit
// byte, or a run start): fixed by the last reset and the digits after it.
BBPE_HD uint32_t digit_phase_out(uint64_t N_, uint64_t DL, uint64_t RS) {
  const int hn = hibit64(~N_), hr = hibit64(RS);
  if (hr > hn) return uint32_t(__builtin_popcountll(DL & above64(hr))) % 3u;
  const uint32_t c = uint32_t(__builtin_popcountll(DL & above64(hn)));
  return c ? (c - 1) % 3u : 3u;
}

// cl100k CR/LF runs.  State per byte: 0 outside a CR/LF run, 1 in a run that
// followed punctuation (pO), 2 in another run (also after a span start SS
// inside it).  st_in: the state entering the word.  E2: the first byte
// after a run of state 1 when it is a non-CR/LF whitespace character's
// first byte (NCL) outside a span start (a match starts there).  Returns
// the state after the word.
BBPE_HD uint32_t cr_runs(uint64_t CR_, uint64_t IN, uint64_t SS, uint64_t pO, uint64_t NCL,
                         uint32_t st_in, uint64_t &E2) {
  const uint64_t starts = CR_ & ~(CR_ << 1);
  uint64_t G = starts & pO & ~SS & ~1ull;
  if ((CR_ & ~SS & 1) && (st_in == 1 || (st_in == 0 && (pO & 1)))) G |= 1;
  G = fill_up(G, CR_ & ~SS);
  const uint64_t after = IN & ~CR_ & NCL & ~SS;
  E2 = (G << 1) & after;
  if (st_in == 1) E2 |= after & 1;
  if (!(CR_ >> 63)) return 0u;
  return (G >> 63) ? 1u : 2u;
}

// The v machine, right to left: v at a byte = "the non-CR/LF whitespace
// continuing here ends at a non-space character of the span".  BRK: span
// breaks (v = 0), NC: non-CR/LF whitespace (v passes through), else v =
// (not whitespace).  v_in: v entering from the next word.  Returns VN, bit
// i = v at byte i+1.
BBPE_HD uint64_t v_next(uint64_t BRK, uint64_t NC, uint64_t WS_, uint32_t v_in) {
  const uint64_t D = BRK | ~NC;           // bytes that set v
  const uint64_t VAL = D & ~BRK & ~WS_;   // ... to 1
  const uint64_t Y = fill_down(VAL, ~D);  // v at each byte, from inside the word
  uint64_t VN = Y >> 1;
  if (v_in) VN |= D ? above64(hibit64(D) - 1) : ~0ull;
  return VN;
}

}  // namespace bbpe
