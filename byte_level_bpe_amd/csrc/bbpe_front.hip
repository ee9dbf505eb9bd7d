// Front half of the encode path on gfx950: UTF-8 validation and character
// counting, tiktoken-safe chunk cuts, special-token matching, and the split
// into pre-tokens.  One wave (64 lanes) per tile; lane l of tile t looks at
// text word 62*t + l - 1 and owns it for 1 <= l <= 62.
#include <hip/hip_runtime.h>

#include "bbpe_classify.h"
#include "bbpe_device.h"
#include "bbpe_kernels.h"
#include "bbpe_word.h"

namespace bbpe {

// ---------------------------------------------------------------------------
// Step 1: classify every byte, report the first invalid UTF-8 sequence, count
// characters per tile, record the last whitespace/non-whitespace change of
// each tile (for the 25,000-character run cuts) and where each segment starts
// in character terms.  Also clears the span masks written by step 3.  Runs
// before the status block is initialised: its error and offset checks go to
// per-tile slots, reduced by step 2.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64) k_count(EncodeArgs a) {
  const int lane = threadIdx.x;
  const uint32_t t = blockIdx.x;
  const int64_t w = int64_t(t) * TILE_WORDS + lane - 1;
  const int64_t base = w * 64;
  const bool owned = lane >= 1 && lane <= int(TILE_WORDS) && w < int64_t(a.n_words);

  Window win;
  load_window(a.text, a.n, base, win);
  uint64_t seg_lo, seg_hi;
  uint32_t seg_at;
  WordMasks m;
  word_setup<true>(a, w, owned, win, seg_lo, seg_hi, seg_at, m);

  const uint64_t segb = ((seg_lo >> 8) | (seg_hi << 56)) & m.valid;  // segment starts in [0,64)
  const uint64_t ws_prev = shfl_up64(m.WS, 1);
  const uint64_t chg = m.lead & (segb | (m.WS ^ shl(m.WS, ws_prev, 1)));

  const uint32_t nch = owned ? uint32_t(__popcll(m.lead)) : 0u;
  const uint32_t incl = wave_incl_sum(nch, lane);
  const uint32_t excl = incl - nch;
  // local (tile) character index of this word's last change, or -1
  int32_t last = -1;
  if (owned && chg) {
    const int hb = 63 - __clzll(chg);
    last = int32_t(excl + uint32_t(__popcll(m.lead & (bit(hb) - 1))));
  }
  // max over lanes
  last = int32_t(wave_reduce(uint32_t(last), uint32_t(INT32_MIN),
                             [](uint32_t x, uint32_t y) { return int32_t(x) > int32_t(y) ? x : y; }));
  if (lane == 63) {
    a.ws.tile_nchar[t] = incl;  // owned lanes only contribute
  }
  if (lane == 0) a.ws.tile_lastchg[t] = last;

  {
    const uint64_t e = wave_reduce(uint64_t((owned && m.err < 64) ? uint64_t(base + m.err) : ~0ull), uint64_t(~0ull),
                                   [](uint64_t x, uint64_t y) { return x < y ? x : y; });
    if (lane == 0) a.ws.tile_err[t] = e;
  }
  if (owned) {
    // segment starts inside this word: their local character index
    uint64_t sb = segb;
    if (sb) {
      // walk segments whose start lies in [base, base+64)
      uint32_t s = seg_at;
      while (s > 0 && a.seg_off[s - 1] >= uint64_t(base)) --s;
      for (; s < a.n_seg && a.seg_off[s] < uint64_t(base) + 64; ++s) {
        if (int64_t(a.seg_off[s]) < base) continue;
        const int j = int(a.seg_off[s] - uint64_t(base));
        a.ws.seg_local[s] = excl + uint32_t(__popcll(m.lead & (bit(j) - 1)));
      }
    }
    a.ws.ss[w] = 0;
    a.ws.spst[w] = 0;
    a.ws.spc[w] = 0;
  }
  // segment offsets must not decrease: every later kernel exits otherwise
  // (k_count itself only reads them to place bits and indexes, all bounded)
  bool bad = false;
  for (uint32_t s = t * 64u + uint32_t(lane); s < a.n_seg; s += gridDim.x * 64u)
    bad = bad || a.seg_off[s + 1] < a.seg_off[s];
  const bool any_bad = __ballot(bad) != 0;
  if (lane == 0) a.ws.tile_bad[t] = any_bad ? 1u : 0u;
}

// ---------------------------------------------------------------------------
// Step 2 (one workgroup): character base of every tile, character index of
// every segment start, and the last run change before every tile.
// ---------------------------------------------------------------------------
// The status block of a non-empty text (first invalid byte, offsets check,
// counters cleared); one thread.
__device__ __forceinline__ void init_status(const EncodeArgs &a, unsigned long long err, bool bad,
                                            unsigned long long n_chars) {
  Status *s = a.ws.status;
  s->err_pos = err;
  s->n_pieces = 0;
  s->n_ids = 0;
  for (uint32_t k = 0; k < ML_COUNT; ++k) s->n_list[k] = 0;
  s->scan_ticket = 0;
  s->scan_fail = 0;
  s->sp_fix = 0;
  s->wc_hits = 0;
  s->err_seg = 0;
  s->n_chars = n_chars;
  // offsets start at 0, end at the text length and never decrease; every
  // later kernel exits when pad2 is set
  const bool ok = !bad && a.seg_off[0] == 0 && a.seg_off[a.n_seg] == a.n;
  s->pad2 = ok ? 0u : 1u;
}

__global__ void __launch_bounds__(1024) k_scan_chars(EncodeArgs a) {
  __shared__ unsigned long long s_sum[33];
  __shared__ long long s_max[33];
  const uint32_t T = a.n_tiles;
  const uint32_t tid = threadIdx.x;
  const uint32_t per = (T + 1023) / 1024;
  const uint32_t t0 = tid * per, t1 = min(T, t0 + per);
  // (each thread's tiles are read FOLD_BATCH at a time, the loads of a
  // batch issued before any is used)
  unsigned long long sum = 0, err = ~0ull;
  uint32_t bad = 0;
  for (uint32_t q = t0; q < t1; q += FOLD_BATCH) {
    uint32_t nc[FOLD_BATCH], bv[FOLD_BATCH];
    unsigned long long ev[FOLD_BATCH];
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
      const bool in = q + j < t1;
      nc[j] = in ? a.ws.tile_nchar[q + j] : 0u;
      ev[j] = in ? a.ws.tile_err[q + j] : ~0ull;
      bv[j] = in ? a.ws.tile_bad[q + j] : 0u;
    }
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
      sum += nc[j];
      err = min(err, ev[j]);
      bad |= bv[j];
    }
  }
  // the status block: first invalid byte, offsets check, counters cleared
  {
    __shared__ unsigned long long s_err[16];
    __shared__ uint32_t s_bad[16];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const unsigned long long o = __shfl_xor(err, d, 64);
      err = o < err ? o : err;
    }
    const bool wbad = __ballot(bad != 0) != 0;
    if ((tid & 63) == 0) {
      s_err[tid / 64] = err;
      s_bad[tid / 64] = wbad ? 1u : 0u;
    }
    __syncthreads();
    if (tid == 0) {
      unsigned long long e = ~0ull;
      uint32_t b = 0;
      for (uint32_t q = 0; q < 16; ++q) {
        e = min(e, s_err[q]);
        b |= s_bad[q];
      }
      init_status(a, e, b != 0, 0);
    }
  }
  unsigned long long total;
  unsigned long long run =
      block_incl_scan<1024>(sum, 0ull, [](unsigned long long x, unsigned long long y) { return x + y; },
                            s_sum, total) - sum;  // exclusive
  long long mx = -1;
  const unsigned long long run0 = run;  // characters before this thread's first tile
  for (uint32_t q = t0; q < t1; q += FOLD_BATCH) {
    uint32_t nc[FOLD_BATCH];
    int32_t lcv[FOLD_BATCH];
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
      const bool in = q + j < t1;
      nc[j] = in ? a.ws.tile_nchar[q + j] : 0u;
      lcv[j] = in ? a.ws.tile_lastchg[q + j] : -1;
    }
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
      if (q + j < t1) a.ws.tile_charbase[q + j] = run;
      if (lcv[j] >= 0) mx = max(mx, (long long)(run + uint32_t(lcv[j])));
      run += nc[j];
    }
  }
  long long mall;
  const long long mincl =
      block_incl_scan<1024>(mx, -1ll, [](long long x, long long y) { return x > y ? x : y; }, s_max, mall);
  // exclusive: the inclusive max of the thread before
  __shared__ long long s_incl[1024];
  s_incl[tid] = mincl;
  __syncthreads();
  long long carry = tid > 0 ? s_incl[tid - 1] : -1;
  unsigned long long base = run0;
  for (uint32_t q = t0; q < t1; q += FOLD_BATCH) {
    uint32_t nc[FOLD_BATCH];
    int32_t lcv[FOLD_BATCH];
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
      const bool in = q + j < t1;
      nc[j] = in ? a.ws.tile_nchar[q + j] : 0u;
      lcv[j] = in ? a.ws.tile_lastchg[q + j] : -1;
    }
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
      if (q + j < t1) a.ws.tile_chgcarry[q + j] = carry;
      if (lcv[j] >= 0) carry = max(carry, (long long)(base + uint32_t(lcv[j])));
      base += nc[j];
    }
  }
  __syncthreads();
  for (uint32_t s = tid; s <= a.n_seg; s += 1024) {
    const uint64_t o = a.seg_off[s];
    if (s == a.n_seg || o >= a.n) {
      a.ws.seg_charstart[s] = total;
    } else {
      const uint32_t tile = uint32_t((o >> 6) / TILE_WORDS);
      a.ws.seg_charstart[s] = a.ws.tile_charbase[tile] + a.ws.seg_local[s];
    }
  }
  if (tid == 0) a.ws.status->n_chars = total;
}

// ---------------------------------------------------------------------------
// Step 3: span structure.  With tiktoken-safe chunking a cut falls before
// every 400,000th character of a segment and, inside each 400,000-character
// window, 25,000 characters after the start of every whitespace or
// non-whitespace run (repeatedly).  In allow_special segments every special
// string found inside one chunk becomes a special piece.  Outputs the masks
// SS (a span starts here: segment start, cut or end of a special), SPST (a
// special starts here) and SPC (byte inside a special).
// ---------------------------------------------------------------------------
// Whether a special starts at text position p (inside the lane's word) and
// ends by seg_end, and its length: the first special whose bytes match.
// The text comes from the wave's bytes staged in LDS (bytes [lo, lo +
// STAGE_BYTES)) and the specials' strings from their copy in LDS (sp_lds,
// when they fit), four bytes at a time; memory is read only past the stage.
// (Compared byte by byte from memory, a match after two near misses cost a
// chain of some twenty dependent loads, 20-25 us for a wave.)
constexpr uint32_t SP_LDS_BYTES = 1024, SP_LDS_MAX = 255;  // strings' bytes, specials
__device__ __forceinline__ uint32_t lds_dword_at(const uint32_t *b32, uint32_t q) {
  return __builtin_amdgcn_alignbyte(b32[(q >> 2) + 1], b32[q >> 2], q & 3u);
}
// SP_LDS: the specials' strings, offsets and heads are in LDS (two
// instances, so that their reads compile to LDS reads rather than to
// generic ones that could address either).
template <bool SP_LDS>
__device__ __forceinline__ bool special_at_staged(const EncodeArgs &a, const uint4 *bytes, int64_t lo,
                                                  const uint32_t *sp_lds, const uint32_t *off_lds,
                                                  const uint32_t *head_lds, const uint32_t *spf_lds,
                                                  uint64_t p, uint64_t seg_end, uint32_t &len) {
  const uint32_t *b32 = reinterpret_cast<const uint32_t *>(bytes);
  if (!a.T.sp_nfirst) {  // (else the candidates are exactly the specials' first bytes)
    const uint32_t b = reinterpret_cast<const uint8_t *>(bytes)[int64_t(p) - lo];
    if (!((spf_lds[b >> 5] >> (b & 31)) & 1)) return false;
  }
  // the text's first four bytes at p, read once and held against each
  // special's first four (head_lds, zero past the special's end) before any
  // longer compare
  const bool head = SP_LDS && int64_t(p) + 8 <= lo + int64_t(STAGE_BYTES);
  const uint32_t tv0 = head ? lds_dword_at(b32, uint32_t(int64_t(p) - lo)) : 0u;
  for (uint32_t k = 0; k < a.T.n_sp; ++k) {
    const uint32_t o = SP_LDS ? off_lds[k] : a.T.sp_off[k];
    const uint32_t L = (SP_LDS ? off_lds[k + 1] : a.T.sp_off[k + 1]) - o;
    if (head) {
      const uint32_t hm = L >= 4 ? 0xFFFFFFFFu : ((1u << (8 * L)) - 1u);
      if ((tv0 ^ head_lds[k]) & hm) continue;
    }
    if (p + L > seg_end) continue;
    bool eq = true;
    for (uint32_t j = head ? 4u : 0u; j < L && eq; j += 4) {
      const uint64_t q = p + j;
      const uint32_t nb = min(4u, L - j);
      uint32_t tv = 0, sv = 0;
      if (int64_t(q) + 8 <= lo + int64_t(STAGE_BYTES)) {
        tv = lds_dword_at(b32, uint32_t(int64_t(q) - lo));
      } else {
        for (uint32_t x = 0; x < nb; ++x) tv |= uint32_t(a.text[q + x]) << (8 * x);
      }
      if (SP_LDS) {
        sv = lds_dword_at(sp_lds, o + j);
      } else {
        for (uint32_t x = 0; x < nb; ++x) sv |= uint32_t(a.T.sp_bytes[o + j + x]) << (8 * x);
      }
      const uint32_t mask = nb == 4 ? 0xFFFFFFFFu : ((1u << (8 * nb)) - 1u);
      eq = ((tv ^ sv) & mask) == 0;
    }
    if (eq) {
      len = L;
      return true;
    }
  }
  return false;
}

// bits [x, 64) of a word that holds positions 0..63; x may be out of range
__device__ __forceinline__ uint64_t from_bit(int x) {
  return x <= 0 ? ~0ull : (x >= 64 ? 0ull : ~(bit(x) - 1));
}

__device__ __forceinline__ unsigned long long wave_incl_sum64(unsigned long long v, int lane) {
  (void)lane;
  return wave_incl_scan(static_cast<uint64_t>(v), uint64_t(0), [](uint64_t x, uint64_t y) { return x + y; });
}

__global__ void __launch_bounds__(64) k_spans(EncodeArgs a) {
  const int lane = threadIdx.x;
  const uint32_t t = blockIdx.x;
  const uint32_t T = a.n_tiles;

  // the character base of this tile, the last run change before it, and
  // (folded) the character base at the start of each tile before it: from
  // step 2's outputs, or, for texts of at most FUSE_TILES tiles, folded here
  // from step 1's per-tile counts (lane l a contiguous run of tiles)
  const bool fold = T <= FUSE_TILES;
  uint64_t tile_base;
  int64_t chg_carry;
  unsigned long long run_excl = 0;  // (fold) characters before lane's first tile
  uint32_t per = 0;
  if (fold) {
    per = (t + 63) / 64;
    const uint32_t q0 = min(t, uint32_t(lane) * per), q1 = min(t, q0 + per);
    // one pass over the lane's run: its character count and its last run
    // change relative to the run's start
    unsigned long long sum = 0;
    long long mx_rel = -1;
    for (uint32_t q = q0; q < q1; q += FOLD_BATCH) {  // loads issued a batch at a time
      int32_t lc[FOLD_BATCH];
      uint32_t nc[FOLD_BATCH];
#pragma unroll
      for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
        const bool in = q + j < q1;
        lc[j] = in ? a.ws.tile_lastchg[q + j] : -1;
        nc[j] = in ? a.ws.tile_nchar[q + j] : 0u;
      }
#pragma unroll
      for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
        if (lc[j] >= 0) mx_rel = max(mx_rel, (long long)(sum + uint32_t(lc[j])));
        sum += nc[j];
      }
    }
    const unsigned long long incl_s = wave_incl_sum64(sum, lane);
    run_excl = incl_s - sum;
    const long long mx = int64_t(wave_reduce(uint64_t(mx_rel >= 0 ? (long long)run_excl + mx_rel : -1),
                                             uint64_t(INT64_MIN),
                                             [](uint64_t x, uint64_t y) { return int64_t(x) > int64_t(y) ? x : y; }));
    tile_base = lane63(uint64_t(incl_s));
    chg_carry = mx;
    // the offsets check over every tile and the status, by block 0 alone:
    // with offsets that decrease somewhere the other blocks' results are
    // never read (every later kernel exits on the status' flag), and every
    // index they form from the offsets is bounded
    uint32_t bad = 0;
    unsigned long long err = ~0ull, nch = 0;
    if (t == 0) {
      for (uint32_t q = uint32_t(lane); q < T; q += 64 * FOLD_BATCH) {  // three loads per tile, batched
        uint32_t bv[FOLD_BATCH], nv[FOLD_BATCH];
        unsigned long long ev[FOLD_BATCH];
#pragma unroll
        for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
          const bool in = q + 64 * j < T;
          bv[j] = in ? a.ws.tile_bad[q + 64 * j] : 0u;
          ev[j] = in ? a.ws.tile_err[q + 64 * j] : ~0ull;
          nv[j] = in ? a.ws.tile_nchar[q + 64 * j] : 0u;
        }
#pragma unroll
        for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
          bad |= bv[j];
          err = min(err, ev[j]);
          nch += nv[j];
        }
      }
    }
    const bool any_bad = __ballot(bad != 0) != 0;
    if (t == 0) {
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        const unsigned long long o = __shfl_xor(err, d, 64);
        err = o < err ? o : err;
        nch += __shfl_xor(nch, d, 64);
      }
      if (lane == 0) init_status(a, err, any_bad, nch);
    }
    if (any_bad || a.seg_off[0] != 0 || a.seg_off[a.n_seg] != a.n) return;
  } else {
    if (a.ws.status->pad2) return;
    tile_base = a.ws.tile_charbase[t];
    chg_carry = a.ws.tile_chgcarry[t];
  }
  const int64_t w = int64_t(t) * TILE_WORDS + lane - 1;
  const int64_t base = w * 64;
  const bool owned = lane >= 1 && lane <= int(TILE_WORDS) && w < int64_t(a.n_words);
  const bool live = lane >= 1 && w < int64_t(a.n_words);  // owned or the right halo

  Window win;
  load_window(a.text, a.n, base, win);
  uint64_t seg_lo, seg_hi;
  uint32_t seg_at;
  WordMasks m;
  word_setup<false>(a, w, owned, win, seg_lo, seg_hi, seg_at, m);
  const uint64_t segb = ((seg_lo >> 8) | (seg_hi << 56)) & m.valid;
  const uint64_t ws_prev = shfl_up64(m.WS, 1);
  const uint64_t chg = m.lead & (segb | (m.WS ^ shl(m.WS, ws_prev, 1)));

  // character index of this word's first character and the last run change
  // before it (lanes 1..63 are contiguous with the tile's character base)
  const uint32_t nch = (lane >= 1) ? uint32_t(__popcll(m.lead)) : 0u;
  const uint32_t incl = wave_incl_sum(nch, lane);
  const uint64_t c0 = tile_base + (incl - nch);
  int64_t lastchg = -1;
  if (lane >= 1 && chg) {
    const int hb = 63 - __clzll(chg);
    lastchg = int64_t(c0 + uint32_t(__popcll(m.lead & (bit(hb) - 1))));
  }
  const int64_t incl_chg = wave_incl_max(lastchg, lane);
  int64_t chg_before = __shfl_up(static_cast<long long>(incl_chg), 1, 64);
  if (lane <= 1) chg_before = -1;
  chg_before = max(chg_before, chg_carry);
  // (fold) character index of the start of this lane's segment, for the
  // lanes that place window cuts: its tile's base plus its index there
  uint64_t segcs_fold = 0;
  if (fold) {
    const uint32_t s = seg_at;
    const uint64_t o = a.seg_off[s];
    const uint32_t tq = o < a.n ? uint32_t((o >> 6) / TILE_WORDS) : t;
    const uint32_t owner = per ? min(63u, tq / per) : 0u;
    const unsigned long long ex = __shfl(run_excl, int(owner), 64);
    if (tq >= t) {
      segcs_fold = tile_base;
    } else {
      unsigned long long b = ex;
      for (uint32_t q = owner * per; q < tq; ++q) b += a.ws.tile_nchar[q];
      segcs_fold = b;
    }
    segcs_fold += (o < a.n) ? a.ws.seg_local[s] : 0u;
  }

  uint64_t cut = 0;
  if (live && (a.flags & BBPE_TIKTOKEN_SAFE) && m.valid) {
    // state at the first character of the word
    uint32_t s = seg_at;
    uint64_t segcs = fold ? segcs_fold : a.ws.seg_charstart[s];
    uint64_t c = c0;
    uint64_t nw, rs, nr;
    {
      const uint64_t off = c > segcs ? c - segcs : 0;
      uint64_t k = (off + 399999) / 400000;
      if (k == 0) k = 1;
      nw = segcs + 400000ull * k;                   // next window boundary >= c
      const uint64_t ws0 = c > segcs ? segcs + 400000ull * ((c - 1 - segcs) / 400000) : segcs;
      rs = max(uint64_t(chg_before < 0 ? 0 : chg_before), ws0);
      if (rs < segcs) rs = segcs;
      uint64_t kk = c > rs ? (c - rs + 24999) / 25000 : 1;
      if (kk == 0) kk = 1;
      nr = rs + 25000ull * kk;                      // next run cut >= c
    }
    // Walking the word's characters in order: a segment start restarts
    // both counts; else the character at nw is a window cut (which restarts
    // the run count); else a run change restarts the run count; else the
    // character at nr is a run cut.  A restart puts the next boundary of
    // its kind at least 25,000 characters on, past the word's end (a word
    // holds at most 64 characters), so each kind of cut falls at most once
    // in a word, at a character found from the counts directly:
    //  * the window cut at character nw, unless a segment starts at or
    //    before it in the word;
    //  * the run cut at character nr, unless a segment start, a run change
    //    or the window cut falls at or before it in the word.
    const uint64_t nlead = uint64_t(__popcll(m.lead));
    const uint64_t segl = segb & m.lead;
    const uint64_t upto_seg = segl ? bit(__ffsll(static_cast<unsigned long long>(segl)) - 1) - 1 : ~0ull;
    uint64_t wcut = 0;
    if (nw - c < nlead) {
      const uint64_t b = bit(nth_set_bit(m.lead, uint32_t(nw - c)));
      wcut = b & upto_seg;  // strictly before the first segment start
    }
    if (nr - c < nlead) {
      const int i = nth_set_bit(m.lead, uint32_t(nr - c));
      const uint64_t through = (i == 63) ? ~0ull : (bit(i + 1) - 1);
      if (((segl | chg | wcut) & through) == 0) cut |= bit(i);
    }
    cut |= wcut;
  }
  const uint64_t brk = segb | cut;                   // span starts known so far
  const uint64_t brk_next = shfl_down64(brk, 1);

  uint64_t sp_st = 0, sp_in = 0, sp_in_next = 0, ss_end = 0, ss_end_next = 0;
  // does any segment overlapping this word allow specials?
  bool any_allow = false;
  if (live && a.T.n_sp > 0 && m.valid) {
    uint32_t s = seg_at;
    any_allow = a.allow[s] != 0;
    for (uint64_t sb = segb; sb && !any_allow; sb &= sb - 1) {
      const uint64_t p = uint64_t(base) + uint64_t(__ffsll(static_cast<unsigned long long>(sb)) - 1);
      while (s + 1 < a.n_seg && a.seg_off[s + 1] <= p) ++s;
      any_allow = a.allow[s] != 0;
    }
  }
  uint64_t cand = 0;
  if (any_allow && !a.T.sp_overlap) {
    // candidates: bytes equal to a special's first byte (an exact per-byte
    // zero test of the window dwords xor the byte), when there are few
    cand = m.lead;
    if (a.T.sp_nfirst) {
      uint64_t fm = 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const uint32_t raw = win.w[4 + q];
        uint32_t z = 0;
        for (uint32_t f = 0; f < a.T.sp_nfirst; ++f) {
          const uint32_t v = raw ^ (((a.T.sp_firsts >> (8 * f)) & 0xFFu) * 0x01010101u);
          z |= ~(((v & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | v | 0x7F7F7F7Fu);  // 0x80 where v's byte is 0
        }
        fm |= gather4(z) << (4 * q);
      }
      cand &= fm;
    }
  }
  // a wave with candidates stages its bytes and the specials' strings in LDS
  if (__ballot(cand != 0)) {
    __shared__ uint4 s_bytes[STAGE_BYTES / 16];
    __shared__ uint32_t s_sp[SP_LDS_BYTES / 4 + 2];
    __shared__ uint32_t s_spo[SP_LDS_MAX + 1];
    __shared__ uint32_t s_head[SP_LDS_MAX];
    __shared__ uint32_t s_spf[8];  // the specials' first bytes, a bitmap
    const int64_t lo = base - int64_t(lane) * 64 - 16;
    stage_window(s_bytes, win, lane);
    if (lane < 8) s_spf[lane] = a.T.sp_first[lane];
    const uint32_t sp_len = a.T.sp_off[a.T.n_sp];
    const bool sp_in_lds = sp_len <= SP_LDS_BYTES && a.T.n_sp <= SP_LDS_MAX;
    if (sp_in_lds) {  // (the blob is padded by 16 bytes)
      const uint32_t *src = reinterpret_cast<const uint32_t *>(a.T.sp_bytes);
      for (uint32_t k = uint32_t(lane); k < sp_len / 4 + 2; k += 64) s_sp[k] = src[k];
      for (uint32_t k = uint32_t(lane); k <= a.T.n_sp; k += 64) s_spo[k] = a.T.sp_off[k];
    }
    __syncthreads();
    if (sp_in_lds) {  // each special's first four bytes, zero past its end
      for (uint32_t k = uint32_t(lane); k < a.T.n_sp; k += 64) {
        const uint32_t L = s_spo[k + 1] - s_spo[k];
        s_head[k] = lds_dword_at(s_sp, s_spo[k]) & (L >= 4 ? 0xFFFFFFFFu : ((1u << (8 * L)) - 1u));
      }
      __syncthreads();
    }
    // this lane's segment: its end and allow flag, read again only when a
    // candidate lies in a later segment
    uint32_t s = seg_at;
    uint64_t seg_next = a.seg_off[s + 1];
    bool allow_s = a.allow[s] != 0;
    while (cand) {
      const int i = __ffsll(static_cast<unsigned long long>(cand)) - 1;
      cand &= cand - 1;
      const uint64_t p = uint64_t(base) + uint64_t(i);
      while (s + 1 < a.n_seg && seg_next <= p) {
        ++s;
        seg_next = a.seg_off[s + 1];
        allow_s = a.allow[s] != 0;
      }
      if (!allow_s) continue;
      uint32_t L;
      const uint64_t seg_end = min(seg_next, a.n);
      if (!(sp_in_lds ? special_at_staged<true>(a, s_bytes, lo, s_sp, s_spo, s_head, s_spf, p, seg_end, L)
                      : special_at_staged<false>(a, s_bytes, lo, s_sp, s_spo, s_head, s_spf, p, seg_end, L)))
        continue;
      // no chunk cut strictly inside the special: bits i+1 .. e-1 over this
      // word and the next
      const int e = i + int(L);  // end, exclusive, in [i+1, i+64]
      const uint64_t lo_in = from_bit(i + 1) & ~from_bit(e), hi_in = ~from_bit(e - 64);
      if ((lo_in & brk) || (hi_in & brk_next)) continue;
      sp_st |= bit(i);
      sp_in |= from_bit(i) & ~from_bit(e);
      sp_in_next |= hi_in;
      if (e < 64) ss_end |= bit(e);
      else ss_end_next |= bit(e - 64);
      cand &= (e >= 64) ? 0 : ~(bit(e) - 1);  // continue after the special
    }
  }
  if (owned) {
    const uint64_t ss = brk | ss_end;
    if (ss) atomicOr(reinterpret_cast<unsigned long long *>(&a.ws.ss[w]), ss);
    if (sp_st) atomicOr(reinterpret_cast<unsigned long long *>(&a.ws.spst[w]), sp_st);
    if (sp_in) atomicOr(reinterpret_cast<unsigned long long *>(&a.ws.spc[w]), sp_in);
    if (w + 1 < int64_t(a.n_words)) {
      if (sp_in_next) atomicOr(reinterpret_cast<unsigned long long *>(&a.ws.spc[w + 1]), sp_in_next);
      if (ss_end_next) atomicOr(reinterpret_cast<unsigned long long *>(&a.ws.ss[w + 1]), ss_end_next);
    }
  }
}

// ---------------------------------------------------------------------------
// Step 3b (special sets whose occurrences can overlap, e.g. "xyx", or
// "<|a|>" with "|>b"): the special pass as the leftmost-first scan of the
// tiktoken page ("Special tokens"): in each chunk of an allow_special
// segment, the leftmost position where a special occurs entirely inside the
// chunk starts one, and the scan resumes after it.  k_spans has written the
// chunk cuts and segment starts (SS) and no specials.  A word's choices
// depend on how far a special chosen in the word before covers it; each
// lane of a tile runs the scan over its word for an incoming coverage, and
// the coverages pass from lane to lane until none changes (one step per
// lane of a chain at most).  The coverage entering a tile comes from a walk
// back from its start to a position that no occurrence covers (its state is
// known there), then the scan forward from that position; a tile whose walk
// back passes SP_WALK_MAX bytes is left to k_specials_fix, which resolves
// such tiles in text order from their predecessors' outgoing coverage.
// (Only long unbroken runs of overlapping occurrences, such as "xyxyxy..."
// for a special "xyx", come near the limit; tiktoken-safe chunking cuts
// them at 25,000 characters.)
// ---------------------------------------------------------------------------
constexpr uint64_t SP_WALK_MAX = 16384;

// Bytes of the 64-byte word at wi that are the first byte of some special.
__device__ __forceinline__ uint64_t sp_first_mask(const EncodeArgs &a, uint64_t wi) {
  uint64_t m = 0;
  const uint64_t b0 = wi * 64;
  for (uint32_t q = 0; q < 16; ++q) {
    const uint64_t addr = b0 + 4 * q;
    if (addr >= a.n) break;
    uint32_t v = 0;
    if (addr + 4 <= a.n) {
      v = *reinterpret_cast<const uint32_t *>(a.text + addr);
    } else {
      for (uint32_t j = 0; addr + j < a.n; ++j) v |= uint32_t(a.text[addr + j]) << (8 * j);
    }
    for (uint32_t j = 0; j < 4 && addr + j < a.n; ++j) {
      const uint32_t b = (v >> (8 * j)) & 0xFFu;
      if ((a.T.sp_first[b >> 5] >> (b & 31)) & 1) m |= uint64_t(1) << (4 * q + j);
    }
  }
  return m;
}

// Length of the special occurring at byte p, or 0: in an allow_special
// segment, entirely inside it, with no chunk cut or segment start strictly
// inside.  (The specials are prefix-free: at most one occurs at p.)
__device__ uint32_t sp_match_len(const EncodeArgs &a, uint64_t p) {
  const uint32_t b0 = a.text[p];
  if (!((a.T.sp_first[b0 >> 5] >> (b0 & 31)) & 1)) return 0;
  uint32_t lo = 0, hi = a.n_seg;  // the segment holding p: the last starting at or before it
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (a.seg_off[mid] <= p) lo = mid + 1;
    else hi = mid;
  }
  const uint32_t seg = lo > 0 ? lo - 1 : 0;
  if (!a.allow[seg]) return 0;
  const uint64_t end = min(a.seg_off[seg + 1], a.n);
  for (uint32_t k = 0; k < a.T.n_sp; ++k) {
    const uint32_t o = a.T.sp_off[k], L = a.T.sp_off[k + 1] - o;
    if (p + L > end) continue;
    bool eq = true;
    for (uint32_t j = 0; j < L && eq; ++j) eq = a.text[p + j] == a.T.sp_bytes[o + j];
    if (!eq) continue;
    for (uint64_t q = p + 1; q < p + L; ++q)
      if ((a.ws.ss[q >> 6] >> (q & 63)) & 1) return 0;
    return L;
  }
  return 0;
}

// The coverage entering byte x: bytes from x on that a special chosen before
// x covers (0: none).  One lane; false when the walk back passes
// SP_WALK_MAX bytes.
__device__ bool sp_cover_into(const EncodeArgs &a, uint64_t x, uint32_t &cov_out) {
  uint64_t s = x;
  for (;;) {
    // an occurrence starting in [s - 63, s) that covers s?
    const uint64_t lo = s >= 63 ? s - 63 : 0;
    uint64_t best = s;
    for (uint64_t wi = lo >> 6; wi * 64 < s; ++wi) {
      uint64_t m = sp_first_mask(a, wi);
      while (m) {
        const uint64_t p = wi * 64 + uint64_t(__ffsll(static_cast<unsigned long long>(m)) - 1);
        m &= m - 1;
        if (p < lo || p >= s || p >= best) continue;
        const uint32_t L = sp_match_len(a, p);
        if (L && p + L > s) best = p;
      }
    }
    if (best == s) break;  // no occurrence covers s: nothing chosen before covers it either
    if (x - best > SP_WALK_MAX) return false;
    s = best;
  }
  uint64_t cov = s;  // the scan forward from s to x
  for (uint64_t wi = s >> 6; wi * 64 < x; ++wi) {
    uint64_t m = sp_first_mask(a, wi);
    while (m) {
      const uint64_t p = wi * 64 + uint64_t(__ffsll(static_cast<unsigned long long>(m)) - 1);
      m &= m - 1;
      if (p < cov || p >= x) continue;
      const uint32_t L = sp_match_len(a, p);
      if (L) cov = p + L;
    }
  }
  cov_out = cov > x ? uint32_t(cov - x) : 0u;
  return true;
}

// The scan over one word entering with `cov` bytes covered: vm marks the
// bytes where a special occurs, lp[b] bit i is bit b of that special's
// length - 1.  Returns the coverage passed on; st, in_lo / in_hi: the
// starts chosen and the bytes inside them in this word / the next.
__device__ __forceinline__ uint32_t sp_scan_word(uint64_t vm, const uint64_t (&lp)[6], uint32_t cov,
                                                 uint64_t &st, uint64_t &in_lo, uint64_t &in_hi) {
  st = in_lo = in_hi = 0;
  uint64_t c = cov >= 64 ? 0 : (vm & ~((uint64_t(1) << cov) - 1));
  while (c) {
    const int i = __ffsll(static_cast<unsigned long long>(c)) - 1;
    uint32_t L = 1;
#pragma unroll
    for (int b = 0; b < 6; ++b) L += uint32_t((lp[b] >> i) & 1) << b;
    const int e = i + int(L);  // in [i + 1, i + 64]
    st |= uint64_t(1) << i;
    const uint64_t from_i = ~((uint64_t(1) << i) - 1);
    in_lo |= e >= 64 ? from_i : (from_i & ((uint64_t(1) << e) - 1));
    if (e > 64) in_hi |= e - 64 >= 64 ? ~0ull : ((uint64_t(1) << (e - 64)) - 1);
    cov = uint32_t(e);
    c = e >= 64 ? 0 : (c & ~((uint64_t(1) << e) - 1));
  }
  return cov > 64 ? cov - 64 : 0u;
}

// The special pass of tile t, given the coverage entering its first owned
// word; writes SPST / SPC and the coverage leaving the tile.  All lanes.
__device__ void sp_tile(const EncodeArgs &a, uint32_t t, int lane, uint32_t cov_first) {
  const int64_t w = int64_t(t) * TILE_WORDS + lane - 1;
  const bool owned = lane >= 1 && lane <= int(TILE_WORDS) && w < int64_t(a.n_words);
  const uint64_t base = owned ? uint64_t(w) * 64 : 0;
  // the word's occurrences, found once
  uint64_t vm = 0, lp[6] = {0, 0, 0, 0, 0, 0};
  if (owned) {
    for (uint64_t c = sp_first_mask(a, uint64_t(w)); c; c &= c - 1) {
      const int i = __ffsll(static_cast<unsigned long long>(c)) - 1;
      const uint32_t L = sp_match_len(a, base + uint64_t(i));
      if (!L) continue;
      vm |= uint64_t(1) << i;
#pragma unroll
      for (int b = 0; b < 6; ++b) lp[b] |= uint64_t(((L - 1) >> b) & 1) << i;
    }
  }
  uint32_t cin = lane == 1 ? cov_first : 0u;
  uint64_t st = 0, in_lo = 0, in_hi = 0;
  uint32_t out = 0;
  for (int it = 0; it < 64; ++it) {  // a chain passes one more lane per step
    out = sp_scan_word(vm, lp, cin, st, in_lo, in_hi);
    uint32_t nin = __shfl_up(out, 1, 64);
    if (lane == 1) nin = cov_first;
    if (lane == 0 || !owned) nin = 0;
    if (!__ballot(nin != cin)) break;
    cin = nin;
  }
  if (owned) {
    if (st) atomicOr(reinterpret_cast<unsigned long long *>(&a.ws.spst[w]), st);
    if (in_lo) atomicOr(reinterpret_cast<unsigned long long *>(&a.ws.spc[w]), in_lo);
    if (in_hi && w + 1 < int64_t(a.n_words))
      atomicOr(reinterpret_cast<unsigned long long *>(&a.ws.spc[w + 1]), in_hi);
  }
  const uint32_t last = __shfl(out, int(TILE_WORDS), 64);
  if (lane == 0) a.ws.tile_sp_eout[t] = last;
}

__global__ void __launch_bounds__(64) k_specials(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  const int lane = threadIdx.x;
  const uint32_t t = blockIdx.x;
  uint32_t cov = 0, ok = 1;
  if (lane == 0 && t > 0) ok = sp_cover_into(a, uint64_t(t) * TILE_BYTES, cov) ? 1u : 0u;
  ok = __shfl(ok, 0, 64);
  cov = __shfl(cov, 0, 64);
  if (lane == 0) a.ws.tile_sp_unres[t] = ok ? 0u : 1u;
  if (!ok) {
    if (lane == 0) atomicOr(&a.ws.status->sp_fix, 1u);
    return;
  }
  sp_tile(a, t, lane, cov);
}

// The tiles k_specials left, in text order, each from the coverage leaving
// the tile before it (one wave; nothing to do unless sp_fix is set).
__global__ void __launch_bounds__(64) k_specials_fix(EncodeArgs a) {
  if (a.ws.status->pad2 || !a.ws.status->sp_fix) return;
  const int lane = threadIdx.x;
  uint32_t prev = 0;  // coverage leaving tile t - 1
  for (uint32_t t = 0; t < a.n_tiles; ++t) {
    if (a.ws.tile_sp_unres[t]) {
      sp_tile(a, t, lane, prev);
      __syncthreads();  // (lane 0's store of the tile's coverage, then everyone's load)
    }
    prev = a.ws.tile_sp_eout[t];
  }
}

}  // namespace bbpe
