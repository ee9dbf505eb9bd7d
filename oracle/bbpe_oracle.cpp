// CPU oracle for the byte-level BPE encode path.  TEST INFRASTRUCTURE ONLY:
// only the test suite, the smoke check and the benchmark's CPU-baseline leg
// may load it.  It shares no code, header, table or helper with the GPU
// library; it is deliberately plain, single-threaded and slow.
//
// What it computes, step by step, with the passage each step follows:
//   * the ranks table maps byte strings to ids, rank = id, all 256 single
//     bytes present (tiktoken deep-dive page, "An encoding is three objects"
//     and "The byte floor");
//   * the text arrives as ordered (text, allow_special) segments and, with
//     tiktoken-safe chunking, each segment is cut into pieces of at most
//     400,000 characters whose whitespace / non-whitespace runs are cut at
//     25,000 characters; each chunk is then encoded as its own text (Baseten
//     page, "Why Kimi K3 tokenization is non-trivial" and "One native call
//     for the whole serving path");
//   * in allow_special segments an exact-string pass finds special tokens
//     before the regex and BPE; elsewhere specials are ordinary text
//     (tiktoken deep-dive page, "Special tokens and the injection nobody
//     plans for");
//   * each span between specials is cut by the split pattern, clause by
//     clause, leftmost-first, with possessive quantifiers (tiktoken deep-dive
//     page, "The split pattern"; the o200k-style letter clause and the
//     r50k digit clause from "r50k, cl100k, o200k");
//   * each pre-token is merged with the parts-vector loop: ranks of adjacent
//     pairs, take the lowest (leftmost on ties), merge, recompute only the two
//     neighbours (tiktoken deep-dive page, "Inside encode");
//   * decode concatenates token bytes (tiktoken deep-dive page, "The byte
//     floor" and "Pitfalls that bite in production").
//
// Readings where the pages are silent are listed where they are applied.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <utility>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// Unicode classes (generated from the regex module, see gen_unicode_props.py)
// ---------------------------------------------------------------------------
struct PropRange { uint32_t lo, hi; int bits; };
const PropRange kProps[] = {
#include "unicode_props.inc"
};
enum { P_L = 1, P_N = 2, P_WS = 4, P_LUT = 8, P_LL = 16, P_LMO = 32, P_M = 64 };

int props(uint32_t cp) {
  size_t lo = 0, hi = sizeof(kProps) / sizeof(kProps[0]);
  while (lo < hi) {
    size_t mid = (lo + hi) / 2;
    if (cp < kProps[mid].lo) hi = mid;
    else if (cp > kProps[mid].hi) lo = mid + 1;
    else return kProps[mid].bits;
  }
  return 0;
}
bool is_letter(uint32_t c) { return props(c) & P_L; }
bool is_number(uint32_t c) { return props(c) & P_N; }
bool is_space(uint32_t c) { return props(c) & P_WS; }
bool is_crlf(uint32_t c) { return c == '\r' || c == '\n'; }
// o200k-style classes: U = Lu Lt Lm Lo M, W = Ll Lm Lo M
bool is_upperish(uint32_t c) { return props(c) & (P_LUT | P_LMO | P_M); }
bool is_lowerish(uint32_t c) { return props(c) & (P_LL | P_LMO | P_M); }

// ---------------------------------------------------------------------------
// UTF-8 (strict: no overlongs, no surrogates, nothing above U+10FFFF)
// ---------------------------------------------------------------------------
struct Chars {
  std::vector<uint32_t> cp;    // code points
  std::vector<size_t> off;     // byte offset of each code point, plus the end
};

// Returns the byte index of the first invalid sequence, or SIZE_MAX.
size_t decode_utf8(const uint8_t *s, size_t n, Chars &out) {
  out.cp.clear();
  out.off.clear();
  size_t i = 0;
  while (i < n) {
    uint8_t b = s[i];
    uint32_t c;
    size_t len;
    if (b < 0x80) { c = b; len = 1; }
    else if (b >= 0xC2 && b <= 0xDF) { c = b & 0x1F; len = 2; }
    else if (b >= 0xE0 && b <= 0xEF) { c = b & 0x0F; len = 3; }
    else if (b >= 0xF0 && b <= 0xF4) { c = b & 0x07; len = 4; }
    else return i;
    if (i + len > n) return i;
    for (size_t k = 1; k < len; ++k) {
      if ((s[i + k] & 0xC0) != 0x80) return i;
      c = (c << 6) | (s[i + k] & 0x3F);
    }
    if (len == 3 && c < 0x800) return i;                 // overlong
    if (len == 4 && (c < 0x10000 || c > 0x10FFFF)) return i;
    if (c >= 0xD800 && c <= 0xDFFF) return i;            // surrogate
    out.cp.push_back(c);
    out.off.push_back(i);
    i += len;
  }
  out.off.push_back(n);
  return SIZE_MAX;
}

// ---------------------------------------------------------------------------
// The split grammars, one clause at a time.  Each clause function returns the
// length (in characters) of its match at position p, or 0 for no match.
// ---------------------------------------------------------------------------
// Reading: the (?i:...) group folds case the way the regex engine does, which
// for the letters s d m t l v e r means ASCII case plus U+017F (long s) as s.
bool ci_is(uint32_t c, char lower) {
  if (c == uint32_t(lower) || c == uint32_t(lower - 'a' + 'A')) return true;
  return lower == 's' && c == 0x17F;
}

struct Span {
  const uint32_t *c;
  size_t n;
  uint32_t at(size_t i) const { return i < n ? c[i] : 0xFFFFFFFFu; }
  bool has(size_t i) const { return i < n; }
};

// '(?i:[sdmt]|ll|ve|re)   -- the alternatives are tried in the printed order
size_t contraction(const Span &s, size_t p) {
  if (!s.has(p) || s.at(p) != '\'') return 0;
  if (s.has(p + 1)) {
    uint32_t a = s.at(p + 1);
    if (ci_is(a, 's') || ci_is(a, 'd') || ci_is(a, 'm') || ci_is(a, 't')) return 2;
  }
  if (s.has(p + 2)) {
    uint32_t a = s.at(p + 1), b = s.at(p + 2);
    if (ci_is(a, 'l') && ci_is(b, 'l')) return 3;
    if (ci_is(a, 'v') && ci_is(b, 'e')) return 3;
    if (ci_is(a, 'r') && ci_is(b, 'e')) return 3;
  }
  return 0;
}

// [^\r\n\p{L}\p{N}]?+\p{L}++
size_t letters_g1(const Span &s, size_t p) {
  size_t j = p;
  if (s.has(j) && !is_crlf(s.at(j)) && !is_letter(s.at(j)) && !is_number(s.at(j))) ++j;
  size_t k = j;
  while (s.has(k) && is_letter(s.at(k))) ++k;
  return k > j ? k - p : 0;
}

// o200k-style letter clause (this project's reading of the one-sentence
// description): [^\r\n\p{L}\p{N}]?+ ( U*+ W++ | U++ W*+ ) (?i:'[sdmt]|'ll|'ve|'re)?+
size_t letters_g2(const Span &s, size_t p) {
  size_t j = p;
  if (s.has(j) && !is_crlf(s.at(j)) && !is_letter(s.at(j)) && !is_number(s.at(j))) ++j;
  size_t end = 0;
  bool ok = false;
  {  // first alternative: U*+ W++
    size_t u = j;
    while (s.has(u) && is_upperish(s.at(u))) ++u;
    size_t w = u;
    while (s.has(w) && is_lowerish(s.at(w))) ++w;
    if (w > u) { end = w; ok = true; }
  }
  if (!ok) {  // second alternative: U++ W*+
    size_t u = j;
    while (s.has(u) && is_upperish(s.at(u))) ++u;
    if (u > j) {
      size_t w = u;
      while (s.has(w) && is_lowerish(s.at(w))) ++w;
      end = w;
      ok = true;
    }
  }
  if (!ok) return 0;
  end += contraction(s, end);  // optional, possessive
  return end - p;
}

// \p{N}{1,3}+
size_t digits(const Span &s, size_t p) {
  size_t k = p;
  while (s.has(k) && k - p < 3 && is_number(s.at(k))) ++k;
  return k - p;
}

// r50k-style digit clause:  ?\p{N}++  (an unbounded run of digits with an
// optional leading space; the space is given back when no digit follows it).
// Reading: the r50k-style grammar is cl100k's pattern with this clause in
// place of \p{N}{1,3}+ (the page names only this change).
size_t digits_r50k(const Span &s, size_t p) {
  size_t j = p;
  if (s.has(j) && s.at(j) == ' ' && s.has(j + 1) && is_number(s.at(j + 1))) ++j;
  size_t k = j;
  while (s.has(k) && is_number(s.at(k))) ++k;
  return k > j ? k - p : 0;
}

bool is_punct(uint32_t c) { return !is_space(c) && !is_letter(c) && !is_number(c); }

//  ?[^\s\p{L}\p{N}]++[\r\n]*+   (the leading " ?" is greedy but may give back)
size_t punct(const Span &s, size_t p) {
  for (int with_space = 1; with_space >= 0; --with_space) {
    size_t j = p;
    if (with_space) {
      if (!(s.has(j) && s.at(j) == ' ')) continue;
      ++j;
    }
    size_t k = j;
    while (s.has(k) && is_punct(s.at(k))) ++k;
    if (k == j) continue;
    while (s.has(k) && is_crlf(s.at(k))) ++k;
    return k - p;
  }
  return 0;
}

size_t ws_run_end(const Span &s, size_t p) {
  size_t k = p;
  while (s.has(k) && is_space(s.at(k))) ++k;
  return k;
}

// \s++$   ($ is the end of the span: each span is its own haystack)
size_t ws_to_end(const Span &s, size_t p) {
  size_t k = ws_run_end(s, p);
  return (k > p && k == s.n) ? k - p : 0;
}

// \s*[\r\n]   (greedy \s* gives back until a CR or LF follows)
size_t ws_then_newline(const Span &s, size_t p) {
  size_t k = ws_run_end(s, p);
  for (size_t t = k; t > p; --t) {
    // \s* takes [p, t-1) and [\r\n] matches at t-1
    if (is_crlf(s.at(t - 1))) return t - p;
  }
  return 0;
}

// \s+(?!\S)
size_t ws_not_before_nonspace(const Span &s, size_t p) {
  size_t k = ws_run_end(s, p);
  for (size_t t = k; t > p; --t) {
    if (t == s.n || is_space(s.at(t))) return t - p;
  }
  return 0;
}

// \s
size_t one_space(const Span &s, size_t p) { return (s.has(p) && is_space(s.at(p))) ? 1 : 0; }

// Length of the match at p, trying the clauses in the pattern's order.
size_t match_at(const Span &s, size_t p, int grammar) {
  size_t m;
  if (grammar == 1) {
    if ((m = letters_g2(s, p))) return m;
  } else {  // cl100k and r50k-style
    if ((m = contraction(s, p))) return m;
    if ((m = letters_g1(s, p))) return m;
  }
  if ((m = grammar == 2 ? digits_r50k(s, p) : digits(s, p))) return m;
  if ((m = punct(s, p))) return m;
  if ((m = ws_to_end(s, p))) return m;
  if ((m = ws_then_newline(s, p))) return m;
  if ((m = ws_not_before_nonspace(s, p))) return m;
  if ((m = one_space(s, p))) return m;
  return 0;
}

// ---------------------------------------------------------------------------
// The encoder
// ---------------------------------------------------------------------------
constexpr int32_t RANK_MAX = INT32_MAX;

struct Oracle {
  std::unordered_map<std::string, int32_t> ranks;
  std::unordered_map<int32_t, std::string> bytes_of;   // decode: id -> bytes
  std::vector<std::pair<std::string, int32_t>> specials;
  int grammar = 0;
  // instrumentation of the merge loop (lookups it performs, excluding the
  // final per-piece read-out, which equals the merge that made the piece)
  uint64_t n_lookups = 0, lookup_key_bytes = 0, n_pieces = 0;
  // when set, pieces are recorded (absolute byte offset, special flag)
  // instead of merged
  std::vector<std::pair<uint64_t, uint8_t>> *piece_sink = nullptr;
  uint64_t sink_base = 0;  // absolute offset of the current segment

  int32_t rank_of(const uint8_t *p, size_t n) const {
    auto it = ranks.find(std::string(reinterpret_cast<const char *>(p), n));
    return it == ranks.end() ? RANK_MAX : it->second;
  }
  int32_t counted_rank(const uint8_t *p, size_t n) {
    ++n_lookups;
    lookup_key_bytes += n + 4;
    return rank_of(p, n);
  }

  // The parts-vector loop for one pre-token of m bytes.
  void merge(const uint8_t *b, size_t m, std::vector<int32_t> &out) {
    ++n_pieces;
    if (m == 0) return;
    std::vector<std::pair<size_t, int32_t>> parts;  // (start, rank of pair at start)
    parts.reserve(m + 1);
    for (size_t i = 0; i <= m; ++i) {
      // entries whose pair would run past the end take the sentinel
      int32_t r = (i + 2 <= m) ? counted_rank(b + i, 2) : RANK_MAX;
      parts.emplace_back(i, r);
    }
    // pair rank of parts[i] and parts[i+1] given the current boundaries
    auto pair_rank = [&](size_t i) -> int32_t {
      if (i + 2 >= parts.size()) return RANK_MAX;
      size_t s = parts[i].first, e = parts[i + 2].first;
      return counted_rank(b + s, e - s);
    };
    while (parts.size() > 1) {
      size_t best = 0;
      int32_t br = RANK_MAX;
      for (size_t i = 0; i < parts.size(); ++i) {
        if (parts[i].second < br) { br = parts[i].second; best = i; }  // strict <: leftmost
      }
      if (br == RANK_MAX) break;
      parts.erase(parts.begin() + long(best) + 1);
      parts[best].second = pair_rank(best);
      if (best > 0) parts[best - 1].second = pair_rank(best - 1);
    }
    for (size_t j = 0; j + 1 < parts.size(); ++j) {
      size_t s = parts[j].first, e = parts[j + 1].first;
      out.push_back(rank_of(b + s, e - s));
    }
  }

  // Split one span (code points with byte offsets) and merge every piece.
  int encode_span(const uint8_t *text, const Chars &ch, size_t c0, size_t c1,
                  std::vector<int32_t> &out) {
    Span s{ch.cp.data() + c0, c1 - c0};
    size_t p = 0;
    while (p < s.n) {
      size_t m = match_at(s, p, grammar);
      if (m == 0) return -1;  // unreachable: every character is covered
      size_t b0 = ch.off[c0 + p], b1 = ch.off[c0 + p + m];
      if (piece_sink) piece_sink->emplace_back(sink_base + b0, 0);
      else merge(text + b0, b1 - b0, out);
      p += m;
    }
    return 0;
  }

  // One chunk: the special pass (when allowed), then spans.
  int encode_chunk(const uint8_t *text, const Chars &ch, size_t c0, size_t c1, bool allow,
                   std::vector<int32_t> &out) {
    size_t b_end = ch.off[c1];
    size_t span_c0 = c0;
    size_t c = c0;
    while (allow && c < c1) {
      // leftmost position where some special occurs entirely inside the chunk;
      // among specials starting there, the longest
      size_t b = ch.off[c];
      const std::pair<std::string, int32_t> *hit = nullptr;
      for (const auto &sp : specials) {
        if (b + sp.first.size() <= b_end &&
            std::memcmp(text + b, sp.first.data(), sp.first.size()) == 0) {
          if (!hit || sp.first.size() > hit->first.size()) hit = &sp;
        }
      }
      if (!hit) { ++c; continue; }
      if (encode_span(text, ch, span_c0, c, out)) return -1;
      if (piece_sink) piece_sink->emplace_back(sink_base + b, 1);
      else out.push_back(hit->second);
      size_t b_after = b + hit->first.size();
      while (c < c1 && ch.off[c] < b_after) ++c;  // specials end on a character boundary
      span_c0 = c;
    }
    return encode_span(text, ch, span_c0, c1, out);
  }
};

// tiktoken-safe chunking of one segment's characters: windows of 400,000
// characters, and inside each window runs of whitespace or of non-whitespace
// cut every 25,000 characters.  "Whitespace" is read as the White_Space
// property (the regex \s class).  Returns chunk boundaries as character
// indices, including 0 and n.
std::vector<size_t> safe_chunks(const Chars &ch) {
  const size_t n = ch.cp.size();
  std::vector<size_t> cuts{0};
  for (size_t w0 = 0; w0 < n; w0 += 400000) {
    size_t w1 = std::min(n, w0 + size_t(400000));
    if (w0 > 0) cuts.push_back(w0);
    bool run_ws = is_space(ch.cp[w0]);
    size_t run_len = 0;
    for (size_t i = w0; i < w1; ++i) {
      bool ws = is_space(ch.cp[i]);
      if (ws != run_ws) {
        run_ws = ws;
        run_len = 1;
      } else {
        ++run_len;
        if (run_len > 25000) {
          cuts.push_back(i);
          run_len = 1;
        }
      }
    }
  }
  if (n > 0) cuts.push_back(n);
  return cuts;
}

}  // namespace

// ---------------------------------------------------------------------------
// C entry points (loaded with ctypes by the tests and the benchmark)
// ---------------------------------------------------------------------------
extern "C" {

// status: 0 ok, -2 bad table, -3 bad specials
void *oracle_new(const uint8_t *key_bytes, const uint64_t *key_off, const int32_t *ranks,
                 uint32_t n, const uint8_t *sp_bytes, const uint64_t *sp_off,
                 const int32_t *sp_ids, uint32_t ns, int grammar, int *status) {
  Oracle *o = new Oracle;
  o->grammar = grammar;
  *status = (grammar >= 0 && grammar <= 2) ? 0 : -2;
  std::unordered_set<int32_t> seen_rank;
  for (uint32_t i = 0; i < n; ++i) {
    std::string k(reinterpret_cast<const char *>(key_bytes + key_off[i]),
                  key_off[i + 1] - key_off[i]);
    if (k.empty() || ranks[i] < 0 || !o->ranks.emplace(k, ranks[i]).second ||
        !seen_rank.insert(ranks[i]).second) {
      *status = -2;
    }
    o->bytes_of[ranks[i]] = k;
  }
  for (int b = 0; b < 256; ++b) {  // the byte floor
    if (!o->ranks.count(std::string(1, char(b)))) *status = -2;
  }
  for (uint32_t i = 0; i < ns; ++i) {
    std::string s(reinterpret_cast<const char *>(sp_bytes + sp_off[i]), sp_off[i + 1] - sp_off[i]);
    Chars tmp;
    if (s.empty() || seen_rank.count(sp_ids[i]) || o->bytes_of.count(sp_ids[i]) ||
        decode_utf8(reinterpret_cast<const uint8_t *>(s.data()), s.size(), tmp) != SIZE_MAX)
      *status = -3;
    o->specials.emplace_back(s, sp_ids[i]);
    o->bytes_of[sp_ids[i]] = s;
  }
  for (size_t i = 0; i < o->specials.size(); ++i)
    for (size_t j = 0; j < o->specials.size(); ++j) {
      const std::string &a = o->specials[i].first, &b = o->specials[j].first;
      if (i != j && b.size() >= a.size() && b.compare(0, a.size(), a) == 0) *status = -3;
    }
  return o;
}

void oracle_free(void *h) { delete static_cast<Oracle *>(h); }

void oracle_counters(void *h, uint64_t *lookups, uint64_t *key_bytes, uint64_t *pieces) {
  Oracle *o = static_cast<Oracle *>(h);
  *lookups = o->n_lookups;
  *key_bytes = o->lookup_key_bytes;
  *pieces = o->n_pieces;
}

void oracle_reset_counters(void *h) {
  Oracle *o = static_cast<Oracle *>(h);
  o->n_lookups = o->lookup_key_bytes = o->n_pieces = 0;
}

// Encode segments.  Returns 0, -4 (invalid UTF-8: *err_seg, *err_byte set),
// -5 (capacity: *n_ids set to the required count) or -1 (internal).
}  // extern "C"

namespace {
int run_segments(Oracle *o, const uint8_t *text, const uint64_t *seg_off, const uint8_t *allow,
                 uint32_t nseg, int safe, std::vector<int32_t> &out, int64_t *id_off,
                 uint64_t *err_seg, uint64_t *err_byte) {
  Chars ch;
  for (uint32_t s = 0; s < nseg; ++s) {
    if (id_off) id_off[s] = int64_t(out.size());
    o->sink_base = seg_off[s];
    const uint8_t *t = text + seg_off[s];
    size_t n = seg_off[s + 1] - seg_off[s];
    size_t bad = decode_utf8(t, n, ch);
    if (bad != SIZE_MAX) {
      *err_seg = s;
      *err_byte = seg_off[s] + bad;
      return -4;
    }
    std::vector<size_t> cuts;
    if (safe) cuts = safe_chunks(ch);
    else cuts = {0, ch.cp.size()};
    for (size_t k = 0; k + 1 < cuts.size(); ++k) {
      if (o->encode_chunk(t, ch, cuts[k], cuts[k + 1], allow[s] != 0, out)) return -1;
    }
  }
  if (id_off) id_off[nseg] = int64_t(out.size());
  return 0;
}
}  // namespace

extern "C" {

int oracle_encode(void *h, const uint8_t *text, const uint64_t *seg_off, const uint8_t *allow,
                  uint32_t nseg, int safe, int32_t *ids, uint64_t cap, int64_t *id_off,
                  uint64_t *n_ids, uint64_t *err_seg, uint64_t *err_byte) {
  Oracle *o = static_cast<Oracle *>(h);
  std::vector<int32_t> out;
  o->piece_sink = nullptr;
  int st = run_segments(o, text, seg_off, allow, nseg, safe, out, id_off, err_seg, err_byte);
  if (st) return st;
  *n_ids = out.size();
  if (out.size() > cap) return -5;
  std::copy(out.begin(), out.end(), ids);
  return 0;
}

// Pieces of whole segments (chunking, specials, split) without merging:
// absolute byte offsets of piece starts and a special flag per piece.
int oracle_pieces(void *h, const uint8_t *text, const uint64_t *seg_off, const uint8_t *allow,
                  uint32_t nseg, int safe, uint64_t *starts, uint8_t *is_special, uint64_t cap,
                  uint64_t *n_out, uint64_t *err_seg, uint64_t *err_byte) {
  Oracle *o = static_cast<Oracle *>(h);
  std::vector<std::pair<uint64_t, uint8_t>> sink;
  std::vector<int32_t> unused;
  o->piece_sink = &sink;
  int st = run_segments(o, text, seg_off, allow, nseg, safe, unused, nullptr, err_seg, err_byte);
  o->piece_sink = nullptr;
  if (st) return st;
  *n_out = sink.size();
  if (sink.size() > cap) return -5;
  for (size_t i = 0; i < sink.size(); ++i) {
    starts[i] = sink[i].first;
    is_special[i] = sink[i].second;
  }
  return 0;
}

// Split one span into pre-tokens; writes byte offsets of piece starts.
int oracle_split(void *h, const uint8_t *text, uint64_t n, uint64_t *starts, uint64_t cap,
                 uint64_t *n_out) {
  Oracle *o = static_cast<Oracle *>(h);
  Chars ch;
  if (decode_utf8(text, n, ch) != SIZE_MAX) return -4;
  Span s{ch.cp.data(), ch.cp.size()};
  size_t p = 0, k = 0;
  while (p < s.n) {
    size_t m = match_at(s, p, o->grammar);
    if (m == 0) return -1;
    if (k < cap) starts[k] = ch.off[p];
    ++k;
    p += m;
  }
  *n_out = k;
  return k > cap ? -5 : 0;
}

// tiktoken-safe chunk boundaries of one segment, as byte offsets (0 and n included).
int oracle_chunks(const uint8_t *text, uint64_t n, uint64_t *cuts, uint64_t cap, uint64_t *n_out) {
  Chars ch;
  if (decode_utf8(text, n, ch) != SIZE_MAX) return -4;
  std::vector<size_t> c = safe_chunks(ch);
  if (c.empty()) c = {0};
  *n_out = c.size();
  if (c.size() > cap) return -5;
  for (size_t i = 0; i < c.size(); ++i) cuts[i] = ch.off[c[i]];
  return 0;
}

// Merge one pre-token (any bytes).
int oracle_merge(void *h, const uint8_t *piece, uint64_t n, int32_t *ids, uint64_t cap,
                 uint64_t *n_out) {
  Oracle *o = static_cast<Oracle *>(h);
  std::vector<int32_t> out;
  o->merge(piece, n, out);
  *n_out = out.size();
  if (out.size() > cap) return -5;
  std::copy(out.begin(), out.end(), ids);
  return 0;
}

// Decode ids to bytes.  Returns 0, -6 (unknown id; *out_len = its index) or
// -5 (capacity; *out_len = required bytes).
int oracle_decode(void *h, const int32_t *ids, uint64_t n, uint8_t *out, uint64_t cap,
                  uint64_t *out_len) {
  Oracle *o = static_cast<Oracle *>(h);
  std::string s;
  for (uint64_t i = 0; i < n; ++i) {
    auto it = o->bytes_of.find(ids[i]);
    if (it == o->bytes_of.end()) { *out_len = i; return -6; }
    s += it->second;
  }
  *out_len = s.size();
  if (s.size() > cap) return -5;
  std::memcpy(out, s.data(), s.size());
  return 0;
}

}  // extern "C"
