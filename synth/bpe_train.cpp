// Plain greedy byte-pair-encoding trainer used to make the synthetic rank
// tables.  It is a data generator, not part of the encoder: it takes a list
// of (pre-token bytes, count) pairs and repeatedly merges the most frequent
// adjacent pair of symbols until the table holds the requested number of
// entries.
//
// Table conventions (tiktoken's "rank is the id" format, as the tiktoken
// deep-dive page describes under "An encoding is three objects"):
//   * the 256 single bytes are present, at the ranks given by a caller
//     supplied permutation of 0..255;
//   * every merge creates the next rank, 256, 257, ...;
//   * on equal pair counts the pair with the smaller (left rank, right rank)
//     wins, so the table is a deterministic function of the input;
//   * a merge whose byte string already exists as a token reuses that token
//     and takes no new rank; pairs whose bytes would exceed max_len are never
//     merged.
//
// I/O (binary, little endian):
//   words file: repeated { u32 count; u32 len; u8 bytes[len]; }
//   output:     repeated { u32 rank; u32 len; u8 bytes[len]; } in rank order
//
// usage: bpe_train <words> <out> <n_ranks> <max_len> <perm: 256 comma-separated ints>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <queue>
#include <string>
#include <unordered_map>
#include <vector>

namespace {

struct Word {
  std::vector<int32_t> sym;
  int64_t cnt;
  uint32_t stamp = 0;
};

inline uint64_t pkey(int32_t a, int32_t b) {
  return (uint64_t(uint32_t(a)) << 32) | uint32_t(b);
}

struct HeapItem {
  int64_t cnt;
  int32_t a, b;
  bool operator<(const HeapItem &o) const {  // max-heap on cnt, then min (a,b)
    if (cnt != o.cnt) return cnt < o.cnt;
    if (a != o.a) return a > o.a;
    return b > o.b;
  }
};

bool read_words(const char *path, std::vector<Word> &words) {
  FILE *f = std::fopen(path, "rb");
  if (!f) return false;
  uint32_t hdr[2];
  std::vector<uint8_t> buf;
  while (std::fread(hdr, 4, 2, f) == 2) {
    buf.resize(hdr[1]);
    if (hdr[1] && std::fread(buf.data(), 1, hdr[1], f) != hdr[1]) { std::fclose(f); return false; }
    Word w;
    w.cnt = hdr[0];
    w.sym.reserve(hdr[1]);
    for (uint8_t c : buf) w.sym.push_back(c);  // byte values for now
    words.push_back(std::move(w));
  }
  std::fclose(f);
  return true;
}

}  // namespace

int main(int argc, char **argv) {
  if (argc != 6) {
    std::fprintf(stderr, "usage: %s words out n_ranks max_len perm\n", argv[0]);
    return 2;
  }
  const int64_t n_ranks = std::atoll(argv[3]);
  const size_t max_len = size_t(std::atoll(argv[4]));
  std::vector<int32_t> perm;
  {
    const char *p = argv[5];
    while (*p) {
      perm.push_back(int32_t(std::strtol(p, const_cast<char **>(&p), 10)));
      if (*p == ',') ++p;
    }
  }
  if (perm.size() != 256) { std::fprintf(stderr, "perm must have 256 entries\n"); return 2; }

  std::vector<Word> words;
  if (!read_words(argv[1], words)) { std::fprintf(stderr, "cannot read words\n"); return 1; }

  // tokens by rank
  std::vector<std::string> tok(256);
  std::unordered_map<std::string, int32_t> index;
  for (int b = 0; b < 256; ++b) {
    tok[perm[b]] = std::string(1, char(b));
  }
  for (int r = 0; r < 256; ++r) index[tok[r]] = r;
  for (auto &w : words)
    for (auto &s : w.sym) s = perm[s];

  std::unordered_map<uint64_t, int64_t> cnt;
  std::unordered_map<uint64_t, std::vector<uint32_t>> where;
  cnt.reserve(1 << 22);
  where.reserve(1 << 22);
  for (uint32_t wi = 0; wi < words.size(); ++wi) {
    const auto &s = words[wi].sym;
    for (size_t i = 0; i + 1 < s.size(); ++i) {
      uint64_t k = pkey(s[i], s[i + 1]);
      cnt[k] += words[wi].cnt;
      auto &v = where[k];
      if (v.empty() || v.back() != wi) v.push_back(wi);
    }
  }
  std::priority_queue<HeapItem> heap;
  for (auto &kv : cnt)
    heap.push({kv.second, int32_t(kv.first >> 32), int32_t(kv.first & 0xffffffffu)});

  int64_t next_rank = 256;
  uint32_t stamp = 0;
  std::unordered_map<uint64_t, int64_t> delta;
  while (next_rank < n_ranks) {
    if (heap.empty()) {
      std::fprintf(stderr, "ran out of pairs at rank %lld\n", (long long)next_rank);
      return 3;
    }
    HeapItem top = heap.top();
    heap.pop();
    uint64_t key = pkey(top.a, top.b);
    auto it = cnt.find(key);
    if (it == cnt.end() || it->second != top.cnt || top.cnt <= 0) continue;  // stale
    const std::string merged = tok[top.a] + tok[top.b];
    if (merged.size() > max_len) continue;
    int32_t t;
    auto ex = index.find(merged);
    if (ex != index.end()) {
      t = ex->second;
    } else {
      t = int32_t(next_rank++);
      tok.push_back(merged);
      index[merged] = t;
    }
    ++stamp;
    delta.clear();
    std::vector<uint32_t> wl;
    wl.swap(where[key]);
    for (uint32_t wi : wl) {
      Word &w = words[wi];
      if (w.stamp == stamp) continue;
      w.stamp = stamp;
      auto &s = w.sym;
      bool hit = false;
      for (size_t i = 0; i + 1 < s.size();) {
        if (s[i] == top.a && s[i + 1] == top.b) {
          hit = true;
          if (i > 0) delta[pkey(s[i - 1], s[i])] -= w.cnt;
          if (i + 2 < s.size()) delta[pkey(s[i + 1], s[i + 2])] -= w.cnt;
          delta[key] -= w.cnt;
          s[i] = t;
          s.erase(s.begin() + long(i) + 1);
          if (i > 0) {
            uint64_t k2 = pkey(s[i - 1], s[i]);
            delta[k2] += w.cnt;
            auto &v = where[k2];
            if (v.empty() || v.back() != wi) v.push_back(wi);
          }
          if (i + 1 < s.size()) {
            uint64_t k2 = pkey(s[i], s[i + 1]);
            delta[k2] += w.cnt;
            auto &v = where[k2];
            if (v.empty() || v.back() != wi) v.push_back(wi);
          }
          ++i;
        } else {
          ++i;
        }
      }
      (void)hit;
    }
    for (auto &kv : delta) {
      if (kv.second == 0) continue;
      int64_t &c = cnt[kv.first];
      c += kv.second;
      if (c > 0) heap.push({c, int32_t(kv.first >> 32), int32_t(kv.first & 0xffffffffu)});
    }
    cnt.erase(key);
  }

  FILE *out = std::fopen(argv[2], "wb");
  if (!out) return 1;
  for (size_t r = 0; r < tok.size(); ++r) {
    uint32_t hdr[2] = {uint32_t(r), uint32_t(tok[r].size())};
    std::fwrite(hdr, 4, 2, out);
    std::fwrite(tok[r].data(), 1, tok[r].size(), out);
  }
  std::fclose(out);
  return 0;
}
