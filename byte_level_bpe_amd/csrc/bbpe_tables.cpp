// Host half of the library: table validation, the device table image,
// decode, and the small C entry points that need no GPU.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/bbpe.h"
#include "bbpe_internal.h"
#include "bbpe_tokenizer.h"

namespace {
#include "unicode_classes.inc"
}

using bbpe::ImageLayout;
using bbpe::Slot;

namespace bbpe {

uint64_t hash_key(const uint8_t *p, uint32_t len) {
  uint64_t h = hash_seed(len);
  for (uint32_t i = 0; i < len; i += 8) {
    uint64_t w = 0;
    uint32_t k = std::min<uint32_t>(8, len - i);
    for (uint32_t j = 0; j < k; ++j) w |= uint64_t(p[i + j]) << (8 * j);
    h = hash_step(h, w);
  }
  return h;
}

}  // namespace bbpe

namespace {

bool valid_utf8(const std::string &s) {
  size_t i = 0, n = s.size();
  const uint8_t *p = reinterpret_cast<const uint8_t *>(s.data());
  while (i < n) {
    uint8_t b = p[i];
    size_t len;
    uint32_t c;
    if (b < 0x80) { ++i; continue; }
    if (b >= 0xC2 && b <= 0xDF) { len = 2; c = b & 0x1F; }
    else if (b >= 0xE0 && b <= 0xEF) { len = 3; c = b & 0x0F; }
    else if (b >= 0xF0 && b <= 0xF4) { len = 4; c = b & 0x07; }
    else return false;
    if (i + len > n) return false;
    for (size_t k = 1; k < len; ++k) {
      if ((p[i + k] & 0xC0) != 0x80) return false;
      c = (c << 6) | (p[i + k] & 0x3F);
    }
    if ((len == 3 && c < 0x800) || (len == 4 && (c < 0x10000 || c > 0x10FFFF)) ||
        (c >= 0xD800 && c <= 0xDFFF))
      return false;
    i += len;
  }
  return true;
}

// True when occurrences of a and b can overlap in some text: a proper suffix
// of a is a proper prefix of b, or b occurs inside a at a non-zero offset.
bool can_overlap(const std::string &a, const std::string &b) {
  for (size_t k = 1; k < a.size() && k < b.size(); ++k)
    if (a.compare(a.size() - k, k, b, 0, k) == 0) return true;
  if (&a != &b)
    for (size_t i = 1; i + b.size() <= a.size(); ++i)
      if (a.compare(i, b.size(), b) == 0) return true;
  return false;
}

// The merge rule on the host, used once per key at load time to find the
// keys whose own bytes merge back to themselves.
bool self_consistent(const std::string &key, int32_t rank,
                     const std::unordered_map<std::string, int32_t> &ranks) {
  const size_t m = key.size();
  if (m == 1) return true;
  std::vector<size_t> start(m + 1);
  for (size_t i = 0; i <= m; ++i) start[i] = i;
  auto pair_rank = [&](size_t i) -> int32_t {  // parts i and i+1
    if (i + 2 >= start.size()) return bbpe::RANK_NONE;
    auto it = ranks.find(key.substr(start[i], start[i + 2] - start[i]));
    return it == ranks.end() ? bbpe::RANK_NONE : it->second;
  };
  std::vector<int32_t> r(m + 1);
  for (size_t i = 0; i <= m; ++i) r[i] = pair_rank(i);
  while (start.size() > 2) {
    size_t best = 0;
    for (size_t i = 1; i + 1 < start.size(); ++i)
      if (r[i] < r[best]) best = i;
    if (r[best] == bbpe::RANK_NONE) break;
    start.erase(start.begin() + long(best) + 1);
    r.erase(r.begin() + long(best) + 1);
    r[best] = pair_rank(best);
    if (best > 0) r[best - 1] = pair_rank(best - 1);
  }
  return start.size() == 2 && ranks.at(key) == rank;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

int build(bbpe_tokenizer *t, std::vector<std::string> &keys, std::vector<int32_t> &rk,
          std::vector<std::string> &sp, std::vector<int32_t> &spid) {
  const uint32_t n = uint32_t(keys.size());
  if (n < 256) return BBPE_E_TABLE;
  std::unordered_map<std::string, int32_t> ranks;
  ranks.reserve(n * 2);
  std::unordered_set<int32_t> seen;
  int32_t max_id = -1;
  uint32_t max_len = 0;
  for (uint32_t i = 0; i < n; ++i) {
    if (keys[i].empty() || keys[i].size() > BBPE_MAX_KEY_BYTES || rk[i] < 0 ||
        rk[i] > int32_t(BBPE_MAX_RANK))
      return BBPE_E_TABLE;
    if (!ranks.emplace(keys[i], rk[i]).second || !seen.insert(rk[i]).second) return BBPE_E_TABLE;
    max_id = std::max(max_id, rk[i]);
    max_len = std::max<uint32_t>(max_len, uint32_t(keys[i].size()));
  }
  for (int b = 0; b < 256; ++b)
    if (!ranks.count(std::string(1, char(b)))) return BBPE_E_TABLE;
  if (sp.size() > BBPE_MAX_SPECIALS) return BBPE_E_SPECIAL;
  std::unordered_set<std::string> sp_seen;
  for (size_t i = 0; i < sp.size(); ++i) {
    if (sp[i].empty() || sp[i].size() > BBPE_MAX_SPECIAL_BYTES || !valid_utf8(sp[i]) ||
        spid[i] < 0 || seen.count(spid[i]) || !sp_seen.insert(sp[i]).second)
      return BBPE_E_SPECIAL;
    seen.insert(spid[i]);
    max_id = std::max(max_id, spid[i]);
  }
  bool overlap = false;
  for (size_t i = 0; i < sp.size(); ++i)
    for (size_t j = 0; j < sp.size(); ++j) {
      if (i != j && sp[j].size() >= sp[i].size() && sp[j].compare(0, sp[i].size(), sp[i]) == 0)
        return BBPE_E_SPECIAL;  // prefix
      overlap = overlap || can_overlap(sp[i], sp[j]);
    }

  t->n_ranks = n;
  t->max_id = max_id;
  t->max_key_len = max_len;
  t->sp = sp;
  t->sp_id = spid;

  // decode map
  t->dense = uint64_t(max_id) < (uint64_t(1) << 24);
  if (t->dense) t->dec_dense.assign(size_t(max_id) + 1, ~uint64_t(0));
  auto add_dec = [&](const std::string &s, int32_t id) {
    uint64_t v = (uint64_t(t->dec_blob.size()) << 8) | uint64_t(s.size());
    t->dec_blob.insert(t->dec_blob.end(), s.begin(), s.end());
    if (t->dense) t->dec_dense[size_t(id)] = v;
    else t->dec_sparse[id] = v;
  };
  for (uint32_t i = 0; i < n; ++i) add_dec(keys[i], rk[i]);
  for (size_t i = 0; i < sp.size(); ++i) add_dec(sp[i], spid[i]);

  // merge table entries: every split of a key into two keys
  std::vector<uint64_t> mt_entries;
  for (uint32_t i = 0; i < n; ++i) {
    const std::string &k = keys[i];
    for (size_t c = 1; c < k.size(); ++c) {
      auto l = ranks.find(k.substr(0, c));
      if (l == ranks.end()) continue;
      auto r = ranks.find(k.substr(c));
      if (r == ranks.end()) continue;
      mt_entries.push_back((uint64_t(1) << 63) |
                           (bbpe::mt_key(uint32_t(l->second), uint32_t(r->second)) << bbpe::MT_ID_BITS) |
                           uint64_t(rk[i]));
    }
  }
  uint32_t n_mt = 64, mt_log = 6;  // at most 0.7 entries per bucket of 2
  while (uint64_t(n_mt) * 7 < mt_entries.size() * 10) n_mt <<= 1, ++mt_log;

  // image layout
  uint32_t n_slots = 1024;
  while (n_slots < 2 * n) n_slots <<= 1;
  uint64_t blob_bytes = 0;
  for (auto &k : keys) blob_bytes += k.size();
  if (blob_bytes + 16 > bbpe::MAX_BLOB) return BBPE_E_TABLE;
  uint64_t sp_bytes = 0;
  for (auto &s : sp) sp_bytes += s.size();
  ImageLayout L{};
  uint64_t o = 0;
  L.slots = o; o = align256(o + uint64_t(n_slots) * sizeof(Slot));
  L.ext = o; o = align256(o + uint64_t(n_slots) * 8);
  L.blob = o; o = align256(o + blob_bytes + 16);
  L.pair = o; o = align256(o + 65536 * 4);
  L.atom = o; o = align256(o + 256 * 4);
  L.inner = o; o = align256(o + 65536 / 8);
  L.uni1 = o; o = align256(o + sizeof(kUniStage1));
  L.uni2 = o; o = align256(o + sizeof(kUniStage2));
  L.sp_bytes = o; o = align256(o + sp_bytes + 16);
  L.sp_off = o; o = align256(o + 4 * (sp.size() + 1));
  L.sp_id = o; o = align256(o + 4 * (sp.size() + 1));
  L.mt = o; o = align256(o + uint64_t(n_mt) * bbpe::MT_BUCKET * 8);
  L.k3 = o; o = align256(o + (uint64_t(1) << 24) / 8);
  L.q4 = o; o = align256(o + (uint64_t(1) << 24) / 8);
  int32_t max_rank = 0;
  for (uint32_t i = 0; i < n; ++i) max_rank = std::max(max_rank, rk[i]);
  L.dec = o; o = align256(o + 8 * (uint64_t(max_rank) + 1));
  L.dblob = o; o = align256(o + t->dec_blob.size() + 16);
  L.dsp = o; o = align256(o + 16 * (sp.size() + 1));
  L.total = o;
  L.n_slots = n_slots;
  L.n_mt_buckets = n_mt;
  t->layout = L;
  t->image.assign(L.total, 0);
  uint8_t *img = t->image.data();

  Slot *slots = reinterpret_cast<Slot *>(img + L.slots);
  uint64_t *ext = reinterpret_cast<uint64_t *>(img + L.ext);
  for (uint32_t i = 0; i < n_slots; ++i) slots[i] = Slot{0, 0, -1};
  uint8_t *blob = img + L.blob;
  uint64_t boff = 0;
  uint32_t n_self = 0;
  for (uint32_t i = 0; i < n; ++i) {
    const std::string &k = keys[i];
    const uint8_t *kp = reinterpret_cast<const uint8_t *>(k.data());
    memcpy(blob + boff, kp, k.size());
    uint64_t k8 = 0, k8b = 0;
    for (size_t j = 0; j < k.size() && j < 8; ++j) k8 |= uint64_t(kp[j]) << (8 * j);
    for (size_t j = 8; j < k.size() && j < 16; ++j) k8b |= uint64_t(kp[j]) << (8 * (j - 8));
    bool self = self_consistent(k, rk[i], ranks);
    n_self += self;
    uint32_t meta = uint32_t(k.size()) | (self ? bbpe::META_SELF : 0u) |
                    (uint32_t(boff) << bbpe::META_OFF_SHIFT);
    uint64_t h = bbpe::hash_key(kp, uint32_t(k.size()));
    uint32_t idx = uint32_t(h) & (n_slots - 1);
    while (slots[idx].rank >= 0) idx = (idx + 1) & (n_slots - 1);
    slots[idx] = Slot{k8, meta, rk[i]};
    ext[idx] = k8b;
    boff += k.size();
  }
  t->n_self_consistent = n_self;
  int32_t *pair = reinterpret_cast<int32_t *>(img + L.pair);
  for (int i = 0; i < 65536; ++i) pair[i] = bbpe::RANK_NONE;
  int32_t *atom = reinterpret_cast<int32_t *>(img + L.atom);
  // byte pairs that occur inside some key: a merge across any other pair is
  // impossible, because the merged part would be a key containing it
  uint32_t *inner = reinterpret_cast<uint32_t *>(img + L.inner);
  for (uint32_t i = 0; i < n; ++i) {
    const std::string &k = keys[i];
    for (size_t j = 0; j + 1 < k.size(); ++j) {
      const uint32_t pr = uint32_t(uint8_t(k[j])) * 256u + uint8_t(k[j + 1]);
      inner[pr >> 5] |= 1u << (pr & 31);
    }
  }
  for (uint32_t i = 0; i < n; ++i) {
    const std::string &k = keys[i];
    if (k.size() == 2) pair[uint8_t(k[0]) * 256 + uint8_t(k[1])] = rk[i];
    if (k.size() == 1) atom[uint8_t(k[0])] = rk[i];
  }
  memcpy(img + L.uni1, kUniStage1, sizeof(kUniStage1));
  memcpy(img + L.uni2, kUniStage2, sizeof(kUniStage2));
  uint8_t *spb = img + L.sp_bytes;
  uint32_t *spo = reinterpret_cast<uint32_t *>(img + L.sp_off);
  int32_t *spi = reinterpret_cast<int32_t *>(img + L.sp_id);
  uint32_t so = 0;
  for (size_t i = 0; i < sp.size(); ++i) {
    spo[i] = so;
    memcpy(spb + so, sp[i].data(), sp[i].size());
    so += uint32_t(sp[i].size());
    spi[i] = spid[i];
  }
  spo[sp.size()] = so;
  // exact 3-byte keys, and the 4-byte substrings of keys (hashed)
  uint32_t *k3 = reinterpret_cast<uint32_t *>(img + L.k3);
  uint32_t *q4 = reinterpret_cast<uint32_t *>(img + L.q4);
  for (uint32_t i = 0; i < n; ++i) {
    const uint8_t *kp = reinterpret_cast<const uint8_t *>(keys[i].data());
    const size_t len = keys[i].size();
    if (len == 3) {
      const uint32_t x = (uint32_t(kp[0]) << 16) | (uint32_t(kp[1]) << 8) | kp[2];
      k3[x >> 5] |= 1u << (x & 31);
    }
    for (size_t j = 0; j + 4 <= len; ++j) {
      const uint32_t x = uint32_t(kp[j]) | (uint32_t(kp[j + 1]) << 8) | (uint32_t(kp[j + 2]) << 16) |
                         (uint32_t(kp[j + 3]) << 24);
      const uint32_t b = bbpe::q4_index(x);
      q4[b >> 5] |= 1u << (b & 31);
    }
  }
  // decode: rank -> (offset, length) into the decode blob; specials by id
  {
    uint64_t *dec = reinterpret_cast<uint64_t *>(img + L.dec);
    memcpy(img + L.dblob, t->dec_blob.data(), t->dec_blob.size());
    auto entry = [&](int32_t id) -> uint64_t {
      return t->dense ? t->dec_dense[size_t(id)] : t->dec_sparse.at(id);
    };
    for (uint32_t i = 0; i < n; ++i) dec[rk[i]] = entry(rk[i]);
    std::vector<std::pair<uint64_t, uint64_t>> dsp;
    for (size_t i = 0; i < sp.size(); ++i) dsp.emplace_back(uint64_t(spid[i]), entry(spid[i]));
    std::sort(dsp.begin(), dsp.end());
    uint64_t *dst = reinterpret_cast<uint64_t *>(img + L.dsp);
    for (size_t i = 0; i < dsp.size(); ++i) {
      dst[2 * i] = dsp[i].first;
      dst[2 * i + 1] = dsp[i].second;
    }
    t->dev_dec_n = uint32_t(max_rank) + 1;
  }
  uint64_t *mt = reinterpret_cast<uint64_t *>(img + L.mt);
  for (uint64_t e : mt_entries) {
    const uint64_t key = (e >> bbpe::MT_ID_BITS) & ((uint64_t(1) << (2 * bbpe::MT_ID_BITS)) - 1);
    uint32_t b = bbpe::mt_bucket(key, 64 - mt_log);
    for (;;) {
      uint64_t *bk = mt + uint64_t(b) * bbpe::MT_BUCKET;
      uint32_t j = 0;
      while (j < bbpe::MT_BUCKET && (bk[j] >> 63)) ++j;
      if (j < bbpe::MT_BUCKET) {
        bk[j] = e;
        break;
      }
      b = (b + 1) & (n_mt - 1);
    }
  }

  bbpe::DevTables &d = t->dev;
  d = bbpe::DevTables{};
  d.slot_mask = n_slots - 1;
  d.mt_mask = n_mt - 1;
  d.dec_n = t->dev_dec_n;
  d.mt_shift = 64 - mt_log;
  d.n_sp = uint32_t(sp.size());
  for (auto &s : sp) d.sp_first[uint8_t(s[0]) >> 5] |= 1u << (uint8_t(s[0]) & 31);
  {
    std::vector<uint8_t> firsts;
    for (auto &s : sp)
      if (std::find(firsts.begin(), firsts.end(), uint8_t(s[0])) == firsts.end())
        firsts.push_back(uint8_t(s[0]));
    d.sp_nfirst = firsts.size() <= 4 ? uint32_t(firsts.size()) : 0u;
    d.sp_firsts = 0;
    for (size_t k = 0; k < firsts.size() && k < 4; ++k) d.sp_firsts |= uint32_t(firsts[k]) << (8 * k);
  }
  d.grammar = t->grammar;
  d.max_key_len = max_len;
  d.sp_overlap = overlap ? 1u : 0u;
  return BBPE_OK;
}

int decode_b64(const char *s, size_t n, std::string &out) {
  static int8_t tbl[256];
  static bool init = false;
  if (!init) {
    memset(tbl, -1, sizeof(tbl));
    const char *a = "ABCDEFGHIJKLMNOPQRSTUVWXYZabcdefghijklmnopqrstuvwxyz0123456789+/";
    for (int i = 0; i < 64; ++i) tbl[uint8_t(a[i])] = int8_t(i);
    init = true;
  }
  out.clear();
  uint32_t acc = 0;
  int bits = 0;
  for (size_t i = 0; i < n; ++i) {
    char c = s[i];
    if (c == '=') break;
    int v = tbl[uint8_t(c)];
    if (v < 0) return -1;
    acc = (acc << 6) | uint32_t(v);
    bits += 6;
    if (bits >= 8) {
      bits -= 8;
      out.push_back(char((acc >> bits) & 0xFF));
    }
  }
  return 0;
}

int collect_specials(const uint8_t *special_bytes, const uint64_t *special_off,
                     const int32_t *special_ids, uint32_t ns, std::vector<std::string> &sp,
                     std::vector<int32_t> &spid) {
  if (ns && (!special_bytes || !special_off || !special_ids)) return BBPE_E_INVALID_ARG;
  for (uint32_t i = 0; i < ns; ++i) {
    if (special_off[i + 1] < special_off[i]) return BBPE_E_SPECIAL;
    sp.emplace_back(reinterpret_cast<const char *>(special_bytes + special_off[i]),
                    size_t(special_off[i + 1] - special_off[i]));
    spid.push_back(special_ids[i]);
  }
  return BBPE_OK;
}

}  // namespace

namespace {
// per host thread: the handle, segment and byte of its last UTF-8 error
struct LastUtf8Error {
  const bbpe_tokenizer *tok = nullptr;
  uint32_t seg = 0;
  uint64_t byte = 0;
};
thread_local LastUtf8Error t_last_err;
}  // namespace

void bbpe::set_last_utf8_error(const bbpe_tokenizer *t, uint32_t seg, uint64_t byte) {
  t_last_err.tok = t;
  t_last_err.seg = seg;
  t_last_err.byte = byte;
}

extern "C" {

int bbpe_load_ranks(const uint8_t *key_bytes, const uint64_t *key_off, const int32_t *ranks,
                    uint32_t n, const uint8_t *special_bytes, const uint64_t *special_off,
                    const int32_t *special_ids, uint32_t ns, int grammar,
                    bbpe_tokenizer **out, uint64_t *device_table_bytes) {
  if (!out || !device_table_bytes || !key_bytes || !key_off || !ranks) return BBPE_E_INVALID_ARG;
  if (grammar != BBPE_GRAMMAR_CL100K && grammar != BBPE_GRAMMAR_O200K_STYLE &&
      grammar != BBPE_GRAMMAR_R50K_STYLE)
    return BBPE_E_INVALID_ARG;
  *out = nullptr;
  std::vector<std::string> keys;
  std::vector<int32_t> rk(ranks, ranks + n);
  keys.reserve(n);
  for (uint32_t i = 0; i < n; ++i) {
    if (key_off[i + 1] < key_off[i]) return BBPE_E_TABLE;
    keys.emplace_back(reinterpret_cast<const char *>(key_bytes + key_off[i]),
                      size_t(key_off[i + 1] - key_off[i]));
  }
  std::vector<std::string> sp;
  std::vector<int32_t> spid;
  int st = collect_specials(special_bytes, special_off, special_ids, ns, sp, spid);
  if (st) return st;
  bbpe_tokenizer *t = new bbpe_tokenizer;
  t->grammar = grammar;
  st = build(t, keys, rk, sp, spid);
  if (st) { delete t; return st; }
  *out = t;
  *device_table_bytes = t->layout.total;
  return BBPE_OK;
}

int bbpe_load_ranks_tiktoken_file(const char *path, const uint8_t *special_bytes,
                                  const uint64_t *special_off, const int32_t *special_ids,
                                  uint32_t ns, int grammar, bbpe_tokenizer **out,
                                  uint64_t *device_table_bytes) {
  if (!path || !out || !device_table_bytes) return BBPE_E_INVALID_ARG;
  if (grammar != BBPE_GRAMMAR_CL100K && grammar != BBPE_GRAMMAR_O200K_STYLE &&
      grammar != BBPE_GRAMMAR_R50K_STYLE)
    return BBPE_E_INVALID_ARG;
  *out = nullptr;
  FILE *f = fopen(path, "rb");
  if (!f) return BBPE_E_TABLE;
  std::vector<std::string> keys;
  std::vector<int32_t> rk;
  char line[1024];
  std::string k;
  while (fgets(line, sizeof(line), f)) {
    size_t len = strlen(line);
    while (len && (line[len - 1] == '\n' || line[len - 1] == '\r')) line[--len] = 0;
    if (!len) continue;
    char *sp = strchr(line, ' ');
    if (!sp || decode_b64(line, size_t(sp - line), k)) { fclose(f); return BBPE_E_TABLE; }
    char *end = nullptr;
    long r = strtol(sp + 1, &end, 10);
    if (end == sp + 1 || *end || r < 0 || r > 0x7fffffffL) { fclose(f); return BBPE_E_TABLE; }
    keys.push_back(k);
    rk.push_back(int32_t(r));
  }
  fclose(f);
  std::vector<std::string> spv;
  std::vector<int32_t> spid;
  int st = collect_specials(special_bytes, special_off, special_ids, ns, spv, spid);
  if (st) return st;
  bbpe_tokenizer *t = new bbpe_tokenizer;
  t->grammar = grammar;
  st = build(t, keys, rk, spv, spid);
  if (st) { delete t; return st; }
  *out = t;
  *device_table_bytes = t->layout.total;
  return BBPE_OK;
}

int bbpe_decode(const bbpe_tokenizer *t, const int32_t *ids, uint64_t n, uint8_t *out,
                uint64_t cap, uint64_t *out_len) {
  if (!t || !out_len || (n && !ids) || (cap && !out)) return BBPE_E_INVALID_ARG;
  uint64_t need = 0;
  for (uint64_t i = 0; i < n; ++i) {
    uint64_t v = ~uint64_t(0);
    int32_t id = ids[i];
    if (id >= 0) {
      if (t->dense) {
        if (uint64_t(id) < t->dec_dense.size()) v = t->dec_dense[size_t(id)];
      } else {
        auto it = t->dec_sparse.find(id);
        if (it != t->dec_sparse.end()) v = it->second;
      }
    }
    if (v == ~uint64_t(0)) { *out_len = i; return BBPE_E_BAD_ID; }
    uint64_t len = v & 0xFF;
    if (need + len <= cap) memcpy(out + need, t->dec_blob.data() + (v >> 8), len);
    need += len;
  }
  *out_len = need;
  return need > cap ? BBPE_E_CAPACITY : BBPE_OK;
}

int bbpe_error_detail(const bbpe_tokenizer *t, uint32_t *segment, uint64_t *byte_offset) {
  if (!t || !segment || !byte_offset) return BBPE_E_INVALID_ARG;
  const bool mine = t_last_err.tok == t;
  *segment = mine ? t_last_err.seg : 0;
  *byte_offset = mine ? t_last_err.byte : 0;
  return BBPE_OK;
}

int bbpe_table_info(const bbpe_tokenizer *t, uint32_t *n_ranks, int32_t *max_id,
                    uint32_t *n_specials, int *grammar) {
  if (!t) return BBPE_E_INVALID_ARG;
  if (n_ranks) *n_ranks = t->n_ranks;
  if (max_id) *max_id = t->max_id;
  if (n_specials) *n_specials = uint32_t(t->sp.size());
  if (grammar) *grammar = t->grammar;
  return BBPE_OK;
}

const char *bbpe_status_str(int s) {
  switch (s) {
    case BBPE_OK: return "ok";
    case BBPE_E_INVALID_ARG: return "invalid argument";
    case BBPE_E_TABLE: return "invalid ranks table";
    case BBPE_E_SPECIAL: return "invalid special tokens";
    case BBPE_E_UTF8: return "invalid UTF-8 in a segment";
    case BBPE_E_CAPACITY: return "ids capacity too small";
    case BBPE_E_BAD_ID: return "id is neither a rank nor a special";
    case BBPE_E_HIP: return "HIP runtime error";
    case BBPE_E_WORKSPACE: return "workspace missing or too small";
    case BBPE_E_STATE: return "tables not uploaded";
    case BBPE_E_NOMEM: return "host allocation failed";
    default: return "unknown status";
  }
}

}  // extern "C"
