// Back half of the encode path on gfx950: the list of merge units, byte-pair
// merging of every unit, and the ordered assembly of ids.
//
// The merge (tiktoken deep-dive page, "Inside encode"): ranks of adjacent
// pairs; repeatedly merge the lowest (leftmost on ties); recompute only the
// two pairs that touch the merged part.  A merged part's id is the rank that
// merged it; a part never merged is a single byte with its atom's rank.
// Every part is a key, so after the first round (byte pairs, from the
// 256x256 pair table) each recomputed pair is looked up by the two part ids
// in the merge table: one bucket load, no key bytes.
//
// k_probe (one thread per unit) settles specials, single bytes and units
// that are keys whose own merges rebuild them; the units left are listed by
// length and merged by k_merge in three tiers:
//   short (<= 32 bytes): one lane per unit, bytes / pair ranks / part ids in
//     registers with static indexing;
//   group (<= 512 bytes): 16, 32 or 64 lanes per unit (<= 128, 256, 512
//     bytes), eight positions per lane in registers, argmin by a reduction
//     over the group;
//   long: one wave per unit, state in global memory, pairs of the least rank
//     merged in batches.
#include <hip/hip_runtime.h>

#include "bbpe_device.h"
#include "bbpe_kernels.h"

namespace bbpe {

// ---------------------------------------------------------------------------
// Unit list
// ---------------------------------------------------------------------------
// one workgroup: exclusive scan of units per tile; the total becomes P
__global__ void __launch_bounds__(1024) k_scan_tiles_np(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  __shared__ uint32_t s_sum[33];
  const uint32_t T = a.n_tiles;
  const uint32_t tid = threadIdx.x;
  const uint32_t per = (T + 1023) / 1024;
  const uint32_t t0 = tid * per, t1 = min(T, t0 + per);
  // (each thread's tiles FOLD_BATCH at a time, a batch's loads issued first)
  uint32_t sum = 0;
  fold_run(a.ws.tile_np, t0, t1, [&](uint32_t, uint32_t c) { sum += c; });
  uint32_t total;
  uint32_t run = block_incl_scan<1024>(sum, 0u, [](uint32_t x, uint32_t y) { return x + y; }, s_sum, total) - sum;
  for (uint32_t q = t0; q < t1; q += FOLD_BATCH) {
    uint32_t c[FOLD_BATCH];
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) c[j] = q + j < t1 ? a.ws.tile_np[q + j] : 0u;
#pragma unroll
    for (uint32_t j = 0; j < FOLD_BATCH; ++j) {
      if (q + j < t1) a.ws.tile_np[q + j] = run;
      run += c[j];
    }
  }
  if (tid == 1023) {
    a.ws.tile_np[T] = total;
    a.ws.status->n_pieces = total;
    a.ws.piece_start[total] = uint32_t(a.n);
  }
}

// unit start offsets, in text order
__global__ void __launch_bounds__(64) k_pieces(EncodeArgs a) {
  const int lane = threadIdx.x;
  const uint32_t t = blockIdx.x;
  const int64_t w = int64_t(t) * TILE_WORDS + lane - 1;
  const bool owned = lane >= 1 && lane <= int(TILE_WORDS) && w < int64_t(a.n_words);
  uint64_t ps = owned ? a.ws.ps[w] : 0;
  const uint32_t c = uint32_t(__popcll(ps));
  const uint32_t incl = wave_incl_sum(c, lane);
  uint32_t tbase;
  if (a.n_tiles <= FUSE_TILES) {
    // units of the tiles before this one (their counts, unscanned)
    uint32_t acc = 0;
    fold_strided(a.ws.tile_np, uint32_t(lane), t, 64u, [&](uint32_t, uint32_t v) { acc += v; });
    tbase = wave_sum(acc);
    if (a.ws.status->pad2) return;  // (checked once the reads above are issued)
    if (t + 1 == a.n_tiles && lane == 63) {
      const uint32_t total = tbase + incl;
      a.ws.status->n_pieces = total;
      a.ws.piece_start[total] = uint32_t(a.n);
    }
  } else {
    tbase = a.ws.tile_np[t];
    if (a.ws.status->pad2) return;
  }
  uint32_t idx = tbase + incl - c;
  const uint32_t base = uint32_t(w * 64);
  while (ps) {
    const int i = __ffsll(static_cast<unsigned long long>(ps)) - 1;
    ps &= ps - 1;
    a.ws.piece_start[idx++] = base + uint32_t(i);
  }
}

// ---------------------------------------------------------------------------
// Rank lookups
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t low_bytes(uint64_t w, uint32_t k) {  // keep k <= 8 bytes
  return k >= 8 ? w : (w & ((uint64_t(1) << (8 * k)) - 1));
}

// Probe the table for a key with hash h, first two words k8 / k8b (zero
// padded) and length len; bytes 16.. (for len > 16) are checked by
// `rest_eq(blob_ptr)`.  The slot and its second key word load together.
__device__ __forceinline__ bool slot_match(const DevTables &T, const Slot &sl, uint64_t e, uint64_t k8,
                                           uint64_t k8b, uint32_t len) {
  return (sl.meta & 0xFFu) == len && sl.k8 == k8 && (len <= 8 || e == k8b);
}
template <typename RestEq>
__device__ __forceinline__ int32_t probe(const DevTables &T, uint64_t h, uint64_t k8, uint64_t k8b,
                                         uint32_t len, uint32_t &meta, RestEq rest_eq) {
  uint32_t idx = uint32_t(h) & T.slot_mask;
  for (;;) {
    const Slot sl = T.slots[idx];
    const uint64_t e = T.ext[idx];
    if (sl.rank < 0) return RANK_NONE;
    if (slot_match(T, sl, e, k8, k8b, len) &&
        (len <= 16 || rest_eq(T.blob + (sl.meta >> META_OFF_SHIFT)))) {
      meta = sl.meta;
      return sl.rank;
    }
    idx = (idx + 1) & T.slot_mask;
  }
}

// Key = text bytes p[0..len).
__device__ __forceinline__ int32_t lookup_text(const DevTables &T, const uint8_t *__restrict__ p,
                                               uint32_t len, uint32_t &meta) {
  if (len > T.max_key_len) return RANK_NONE;
  auto word = [&](uint32_t i) __attribute__((always_inline)) {  // bytes i.. of the key, zero padded
    const uint32_t k = min(8u, len - i);
    uint64_t wv = 0;
    for (uint32_t j = 0; j < k; ++j) wv |= uint64_t(p[i + j]) << (8 * j);
    return wv;
  };
  const uint64_t k8 = word(0), k8b = len > 8 ? word(8) : 0ull;
  uint64_t h = hash_step(hash_seed(len), k8);
  if (len > 8) h = hash_step(h, k8b);
  for (uint32_t i = 16; i < len; i += 8) h = hash_step(h, word(i));
  return probe(T, h, k8, k8b, len, meta, [&](const uint8_t *b) __attribute__((always_inline)) {
    for (uint32_t j = 16; j < len; ++j)
      if (b[j] != p[j]) return false;
    return true;
  });
}

// ---------------------------------------------------------------------------
// Merge table lookups: the rank of bytes(a) + bytes(b) for part ids a, b.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mt_load(const DevTables &T, uint32_t b, uint64_t (&e)[MT_BUCKET]) {
  const ulonglong2 *q = reinterpret_cast<const ulonglong2 *>(T.mt + uint64_t(b) * MT_BUCKET);
#pragma unroll
  for (uint32_t k = 0; k < MT_BUCKET / 2; ++k) {
    const ulonglong2 v = q[k];
    e[2 * k] = v.x;
    e[2 * k + 1] = v.y;
  }
}

// rank in the bucket, or RANK_NONE; `more` when the bucket is full without it
__device__ __forceinline__ int32_t mt_find(const uint64_t (&e)[MT_BUCKET], uint64_t want, bool &more) {
  int32_t r = RANK_NONE;
  bool full = true;
#pragma unroll
  for (uint32_t k = 0; k < MT_BUCKET; ++k) {
    r = (e[k] >> MT_ID_BITS) == want ? int32_t(e[k] & MT_ID_MASK) : r;
    full = full && (e[k] >> 63);
  }
  more = full && r == RANK_NONE;
  return r;
}

// the buckets after a full one
__device__ __attribute__((noinline)) int32_t mt_rest(const DevTables &T, uint32_t b, uint64_t want) {
  for (;;) {
    b = (b + 1) & T.mt_mask;
    uint64_t e[MT_BUCKET];
    mt_load(T, b, e);
    bool more;
    const int32_t r = mt_find(e, want, more);
    if (!more) return r;
  }
}

__device__ __forceinline__ int32_t merge_rank(const DevTables &T, uint32_t a, uint32_t b) {
  const uint64_t k = mt_key(a, b);
  const uint32_t x = mt_bucket(k, T.mt_shift);
  const uint64_t want = (uint64_t(1) << (2 * MT_ID_BITS)) | k;
  uint64_t e[MT_BUCKET];
  mt_load(T, x, e);
  bool more;
  const int32_t r = mt_find(e, want, more);
  return more ? mt_rest(T, x, want) : r;
}

// two lookups (v1 / v2: wanted) with both buckets loaded before either is used
__device__ __forceinline__ void merge_rank2(const DevTables &T, bool v1, uint32_t a1, uint32_t b1,
                                            bool v2, uint32_t a2, uint32_t b2, int32_t &r1,
                                            int32_t &r2) {
  const uint64_t k1 = mt_key(a1, b1), k2 = mt_key(a2, b2);
  const uint32_t x1 = mt_bucket(k1, T.mt_shift), x2 = mt_bucket(k2, T.mt_shift);
  const uint64_t w1 = (uint64_t(1) << (2 * MT_ID_BITS)) | k1;
  const uint64_t w2 = (uint64_t(1) << (2 * MT_ID_BITS)) | k2;
  uint64_t e1[MT_BUCKET] = {}, e2[MT_BUCKET] = {};
  if (v1) mt_load(T, x1, e1);
  if (v2) mt_load(T, x2, e2);
  bool m1, m2;
  r1 = mt_find(e1, w1, m1);
  r2 = mt_find(e2, w2, m2);
  if (v1 && m1) r1 = mt_rest(T, x1, w1);
  if (v2 && m2) r2 = mt_rest(T, x2, w2);
  if (!v1) r1 = RANK_NONE;
  if (!v2) r2 = RANK_NONE;
}

// id of the special whose string is p[0..len)
__device__ __forceinline__ int32_t special_id(const DevTables &T, const uint8_t *p, uint32_t len) {
  for (uint32_t k = 0; k < T.n_sp; ++k) {
    const uint32_t o = T.sp_off[k];
    if (T.sp_off[k + 1] - o != len) continue;
    bool eq = true;
    for (uint32_t j = 0; j < len && eq; ++j) eq = p[j] == T.sp_bytes[o + j];
    if (eq) return T.sp_id[k];
  }
  return -1;  // unreachable: special pieces are exact matches
}

// ---------------------------------------------------------------------------
// Unit bytes in registers: units of at most SK bytes, one lane each.
// ---------------------------------------------------------------------------
template <int SK>
struct UnitBytes {
  static constexpr int NB = SK / 4 + 3;  // dwords, with room for 8-byte slices
  uint32_t d[NB];
  __device__ __forceinline__ uint32_t byte(int j) const { return (d[j >> 2] >> (8 * (j & 3))) & 0xFFu; }
  // bytes a .. a+7 (a dynamic, a + 8 <= 4 * NB)
  __device__ __forceinline__ uint64_t slice8(uint32_t a) const {
    const uint32_t q = a >> 2, o = a & 3u;
    uint32_t x0 = 0, x1 = 0, x2 = 0;
#pragma unroll
    for (int qq = 0; qq + 2 < NB; ++qq) {
      const bool hit = uint32_t(qq) == q;
      x0 = hit ? d[qq] : x0;
      x1 = hit ? d[qq + 1] : x1;
      x2 = hit ? d[qq + 2] : x2;
    }
    const uint32_t lo = __builtin_amdgcn_alignbyte(x1, x0, o);
    const uint32_t hi = __builtin_amdgcn_alignbyte(x2, x1, o);
    return (uint64_t(hi) << 32) | lo;
  }
  __device__ __forceinline__ bool operator==(const UnitBytes &o) const {
    bool eq = true;
#pragma unroll
    for (int q = 0; q < NB; ++q) eq = eq && d[q] == o.d[q];
    return eq;
  }
};

// bytes [s, s+m) of the text, zero beyond m (m <= SK).  The aligned 16-byte
// chunks that hold them are loaded whole (a chunk holding a byte of the
// text lies in that byte's page: the text is 16-byte aligned), at most
// SK/16 + 1 of them, then shifted into place: a few wide loads per unit
// instead of one per dword.
template <int SK>
__device__ __forceinline__ void load_unit(const uint8_t *__restrict__ text, uint64_t n, uint32_t s,
                                          uint32_t m, UnitBytes<SK> &u) {
  constexpr int NB = UnitBytes<SK>::NB;
  constexpr int NC = (SK + 14) / 16 + 1;  // chunks over [s, s + SK) at any offset
  constexpr int NQ = SK / 4;  // dwords that can hold unit bytes
  static_assert(4 * NC >= NQ + 4, "chunks cover the shifted dwords");
  const uint32_t off = s & 15u, sh = off >> 2, ob = off & 3u;
  const uint4 *c = reinterpret_cast<const uint4 *>(text) + (s >> 4);
  uint32_t raw[4 * NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const bool in = 16u * j < off + m && (uint64_t(s >> 4) + j) * 16 < n;
    const uint4 v = in ? c[j] : make_uint4(0, 0, 0, 0);
    raw[4 * j] = v.x;
    raw[4 * j + 1] = v.y;
    raw[4 * j + 2] = v.z;
    raw[4 * j + 3] = v.w;
  }
  // shift by sh dwords: by 2, then by 1
  uint32_t r1[4 * NC], r2[4 * NC];
#pragma unroll
  for (int q = 0; q < 4 * NC; ++q) r1[q] = (sh & 2u) ? (q + 2 < 4 * NC ? raw[q + 2] : 0u) : raw[q];
#pragma unroll
  for (int q = 0; q < 4 * NC; ++q) r2[q] = (sh & 1u) ? (q + 1 < 4 * NC ? r1[q + 1] : 0u) : r1[q];
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    if (q > NQ) {
      u.d[q] = 0u;
      continue;
    }
    const uint32_t v = __builtin_amdgcn_alignbyte(q + 1 < 4 * NC ? r2[q + 1] : 0u, r2[q], ob);
    const int lim = int(m) - 4 * q;
    const uint32_t keep = lim >= 4 ? 0xFFFFFFFFu : (lim <= 0 ? 0u : ((1u << (8 * lim)) - 1));
    u.d[q] = v & keep;
  }
}

template <int SK>
__device__ __forceinline__ void unit_hash(const UnitBytes<SK> &u, uint32_t a, uint32_t len,
                                          uint64_t &h, uint64_t &k8, uint64_t &k8b) {
  // (the first two words are named outside the loop: selecting them inside
  // it let the compiler build a dynamically indexed array in scratch)
  k8 = low_bytes(u.slice8(a), len);
  k8b = len > 8 ? low_bytes(u.slice8(a + 8), len - 8) : 0ull;
  h = hash_step(hash_seed(len), k8);
  if (len > 8) h = hash_step(h, k8b);
  for (uint32_t i = 16; i < len; i += 8) h = hash_step(h, low_bytes(u.slice8(a + i), len - i));
}

// key bytes 16..len of the unit slice [a, a+len) against the blob
template <int SK>
__device__ __forceinline__ bool unit_rest_eq(const UnitBytes<SK> &u, uint32_t a, uint32_t len,
                                             const uint8_t *b) {
  for (uint32_t i = 16; i < len; i += 8) {
    const uint32_t k = min(8u, len - i);
    uint64_t bw = 0;
    for (uint32_t j = 0; j < k; ++j) bw |= uint64_t(b[i + j]) << (8 * j);
    if (bw != low_bytes(u.slice8(a + i), k)) return false;
  }
  return true;
}

__device__ __forceinline__ uint32_t above32(int j) { return ~((2u << j) - 1u); }

// One lane's column of the LDS part-id array [32 positions][64 lanes]: ids
// are below 2^21, kept as a 16-bit low part and an 8-bit high part (6 KB per
// wave instead of 8 KB, which lets more merge waves share a CU).
struct PartCol {
  uint16_t *lo;
  uint8_t *hi;
  __device__ __forceinline__ int32_t get(int j) const {
    return int32_t(uint32_t(lo[64 * j]) | (uint32_t(hi[64 * j]) << 16));
  }
  __device__ __forceinline__ void set(int j, int32_t v) const {
    lo[64 * j] = uint16_t(uint32_t(v));
    hi[64 * j] = uint8_t(uint32_t(v) >> 16);
  }
};

// Merge a unit of 2 <= m <= SK bytes held in registers: pair ranks r[j] and
// part ids pr[j] at every part start j, part starts as the bit mask bnd.
// Writes the ids to out and returns their count.
// atom: the 256 atom ranks (a copy in LDS).  lp: this lane's column of an
// LDS array [32][64] holding the id of the part starting at each position
// (read and written at per-lane positions without select chains).  Pair
// ranks stay in registers as keys (rank << 5 | position, or ~0 for none), so
// the leftmost least rank is one unsigned minimum per position.
template <int SK>
__device__ __forceinline__ uint32_t merge_short(const DevTables &T, const int32_t *atom,
                                                const UnitBytes<SK> &u, uint32_t m, const PartCol &lp,
                                                int32_t *out) {
  uint32_t r[SK];
#pragma unroll
  for (int j = 0; j < SK; ++j) {
    const uint32_t b0 = u.byte(j), b1 = (j + 1 < SK) ? u.byte(j + 1) : 0u;
    const int32_t rk = (uint32_t(j) + 1 < m) ? T.pair[b0 * 256u + b1] : RANK_NONE;
    r[j] = rk == RANK_NONE ? ~0u : (uint32_t(rk) << 5) | uint32_t(j);
    if (uint32_t(j) < m) lp.set(j, atom[b0]);
  }
  uint32_t bnd = (m >= 32) ? 0xFFFFFFFFu : ((1u << m) - 1u);
  for (uint32_t round = 0; round + 1 < m; ++round) {
    uint32_t key = ~0u;
#pragma unroll
    for (int j = 0; j < SK; ++j) key = min(key, r[j]);
    if (key == ~0u) break;
    const int bj = int(key & 31u);
    const int32_t best = int32_t(key >> 5);
    const int k = __ffs(bnd & above32(bj)) - 1;  // the part merged into bj
    bnd &= ~(1u << k);
    const uint32_t after = bnd & above32(bj);
    const uint32_t k2 = after ? uint32_t(__ffs(after) - 1) : m;  // end of the merged part
    const uint32_t before = bnd & ((1u << bj) - 1u);
    const int q = before ? 31 - __clz(before) : -1;
    // the merged part (id best) with its right and left neighbours
    const int32_t id2 = after ? lp.get(int(k2)) : 0;
    const int32_t idq = q >= 0 ? lp.get(q) : 0;
    int32_t nb, nq;
    merge_rank2(T, after != 0, uint32_t(best), uint32_t(id2), q >= 0, uint32_t(idq), uint32_t(best),
                nb, nq);
    lp.set(bj, best);
    const uint32_t kb = nb == RANK_NONE ? ~0u : (uint32_t(nb) << 5) | uint32_t(bj);
    const uint32_t kq = nq == RANK_NONE ? ~0u : (uint32_t(nq) << 5) | uint32_t(q);
#pragma unroll
    for (int j = 0; j < SK; ++j) {
      r[j] = (j == k) ? ~0u : r[j];
      r[j] = (j == bj) ? kb : r[j];
      r[j] = (j == q) ? kq : r[j];
    }
  }
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < SK; ++j)
    if ((bnd >> j) & 1u) out[c++] = lp.get(j);
  return c;
}

// ---------------------------------------------------------------------------
// Word cache of one call.  Units with equal bytes merge to equal ids (the
// merge of a unit depends on its bytes alone), so of all the units of 2-16
// bytes with one byte string only one, its leader, runs the merge loop; the
// others follow it.  k_probe stores each such unit's index in the slot
// chosen by a hash of its bytes (plain stores: the last one wins).  The
// leader of a byte string is the unit its slot holds if that unit has the
// same bytes; otherwise every unit with the string leads itself.  Every
// unit of one byte string reads the same slot, so they all agree on it, and
// the leader finds itself there.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t owner_slot(uint64_t h, uint32_t mask) {
  return uint32_t(h >> 40) & mask;
}
// largest unit index a follower can record (UID_FOLLOW - j must be an int32)
constexpr uint32_t FOLLOW_MAX = uint32_t(UID_FOLLOW - INT32_MIN);

// ---------------------------------------------------------------------------
// Word cache kept across calls (BBPE_KEEP_WORD_CACHE): the ids of units of
// 2-32 bytes that went through the merge loop, by their bytes, for the
// calls that follow (a serving process meets the same words in request
// after request; the per-call cache above only spans one call).  Entries of
// 32 dwords: the unit's bytes zero padded (0-7), meta (8: WC_FULL | length
// << 8 | id count; 0 = empty, WC_BUSY = being written), ids (9-31).  An
// entry sits at most WC_PROBES slots past the slot of its bytes' hash;
// entries are never removed (bbpe_word_cache_clear empties the cache), so
// a probe ends at the first empty slot.  k_probe reads the cache; k_merge
// adds the units it merges (claiming an empty slot with a compare-and-swap,
// then writing it, then marking it full), which later calls see.
// Best-effort: a unit whose slots are busy or taken is not added.
// ---------------------------------------------------------------------------
constexpr uint32_t WC_WORDS = 32, WC_MAX_IDS = 23, WC_PROBES = 4;
constexpr uint32_t WC_FULL = 1u << 31, WC_BUSY = 1u << 30;
__device__ __forceinline__ uint32_t wc_slot(uint64_t h, uint32_t mask) { return uint32_t(h >> 20) & mask; }

template <int SK>
__device__ __forceinline__ bool wc_key_eq(const uint32_t *e, const UnitBytes<SK> &u) {
  const uint4 k0 = reinterpret_cast<const uint4 *>(e)[0], k1 = reinterpret_cast<const uint4 *>(e)[1];
  const uint32_t k[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
  bool eq = true;
#pragma unroll
  for (int q = 0; q < 8; ++q) eq = eq && k[q] == (q < UnitBytes<SK>::NB ? u.d[q] : 0u);
  return eq;
}

// The cached ids of unit i (bytes u, m of them, hash h, text offset s), if
// any: written to tmp_ids and piece_cnt as the merge would.
template <int SK>
__device__ __forceinline__ bool wc_find(const EncodeArgs &a, const UnitBytes<SK> &u, uint32_t m,
                                        uint64_t h, uint32_t s, uint32_t i, uint32_t p0 = 0) {
  const uint32_t home = wc_slot(h, a.wc_mask);
  for (uint32_t p = p0; p < WC_PROBES; ++p) {
    const uint32_t *e = a.wcache + uint64_t((home + p) & a.wc_mask) * WC_WORDS;
    const uint32_t meta = e[8];
    if (!(meta & WC_FULL)) return false;
    if (((meta >> 8) & 63u) != m || !wc_key_eq(e, u)) continue;
    const uint32_t cnt = meta & 63u;
    for (uint32_t j = 0; j < cnt; ++j) a.ws.tmp_ids[s + j] = int32_t(e[9 + j]);
    a.ws.piece_cnt[i] = cnt;
    return true;
  }
  return false;
}

// Add a merged unit (its cnt ids at tmp_ids + s) to the cache.
template <int SK>
__device__ __forceinline__ void wc_put(const EncodeArgs &a, const UnitBytes<SK> &u, uint32_t m,
                                       uint32_t s, uint32_t cnt) {
  if (cnt > WC_MAX_IDS) return;
  uint64_t h, k8, k8b;
  unit_hash(u, 0, m, h, k8, k8b);
  const uint32_t home = wc_slot(h, a.wc_mask);
  for (uint32_t p = 0; p < WC_PROBES; ++p) {
    uint32_t *e = a.wcache + uint64_t((home + p) & a.wc_mask) * WC_WORDS;
    // a plain read first: a repeated word finds itself without an atomic
    const uint32_t cur = e[8];
    if (cur & WC_BUSY) return;
    if (cur & WC_FULL) {
      if (((cur >> 8) & 63u) == m && wc_key_eq(e, u)) return;
      continue;
    }
    const uint32_t old = atomicCAS(e + 8, 0u, WC_BUSY);
    if (old == 0) {
#pragma unroll
      for (int q = 0; q < 8; ++q) e[q] = q < UnitBytes<SK>::NB ? u.d[q] : 0u;
      for (uint32_t j = 0; j < cnt; ++j) e[9 + j] = uint32_t(a.ws.tmp_ids[s + j]);
      __threadfence();
      atomicExch(e + 8, WC_FULL | (m << 8) | cnt);
      return;
    }
    if (old & WC_BUSY) return;                                  // another unit is writing here
    if (((old >> 8) & 63u) == m && wc_key_eq(e, u)) return;    // already cached
  }
}

// ---------------------------------------------------------------------------
// Probe pass: one thread per unit.
// ---------------------------------------------------------------------------
constexpr uint32_t WNS = 8;                // positions per lane in the group tiers
constexpr uint32_t WAVE_MAX = 64 * WNS;    // longest unit the group tiers hold
constexpr uint32_t GROUP_PACK_MIN = 4096;  // group units above which several share a wave
constexpr uint32_t FEW32_MAX = 256;        // 17-32-byte units taken 32 lanes each up to this

// Continue a probe whose first slot (sl, e at index idx) is already loaded.
template <typename RestEq>
__device__ __forceinline__ int32_t probe_from(const DevTables &T, uint32_t idx, Slot sl, uint64_t e,
                                              uint64_t k8, uint64_t k8b, uint32_t len,
                                              uint32_t &meta, RestEq rest_eq) {
  for (;;) {
    if (sl.rank < 0) return RANK_NONE;
    if (slot_match(T, sl, e, k8, k8b, len) &&
        (len <= 16 || rest_eq(T.blob + (sl.meta >> META_OFF_SHIFT)))) {
      meta = sl.meta;
      return sl.rank;
    }
    idx = (idx + 1) & T.slot_mask;
    sl = T.slots[idx];
    e = T.ext[idx];
  }
}

// Every unit: specials, single bytes and units that are keys whose own
// merges rebuild them get their id here; the rest are listed for the merge
// kernels by length class.  Each thread takes PROBE_U (4) units and issues the
// loads of all of them (offsets, then bytes and special bits, then the
// first hash slot) before it resolves any, so that one wave keeps several
// units' memory chains in flight.  Each block gathers its list entries in
// LDS (one array, grouped by class) and reserves room in the global lists
// with one atomic per class.
// (Texts under PROBE_SMALL bytes take one unit per thread instead: with few
// units, the four serial resolutions of a thread are the kernel's length.
// Texts from PROBE_MID bytes take two: there twice the waves hide the
// memory chains better than the four side by side in one thread -- 11.5 MB
// of short requests 331 -> 321 us per call, 64 MiB 1.74 -> 1.69 ms -- while
// 4.2 MB is faster with four, 164 against 168 us.)
template <uint32_t PROBE_U, bool WC>
__device__ __forceinline__ void probe_body(const EncodeArgs &a) {
  constexpr uint32_t PROBE_CHUNK = PROBE_BLOCK * PROBE_U;
  if (a.ws.status->pad2) return;
  Status *st = a.ws.status;
  const uint32_t P = uint32_t(st->n_pieces);
  const DevTables &T = a.T;
  __shared__ unsigned int s_cnt[ML_COUNT], s_base[ML_COUNT], s_off[ML_COUNT], s_cur[ML_COUNT];
  __shared__ uint32_t s_list[PROBE_CHUNK];
  __shared__ int32_t s_atom[256];
  if (threadIdx.x < 256) s_atom[threadIdx.x] = T.atom[threadIdx.x];
  // the tile states of k_assemble's scan start unpublished
  for (uint32_t k = blockIdx.x * PROBE_BLOCK + threadIdx.x; k <= P / ASM_UNITS; k += gridDim.x * PROBE_BLOCK)
    a.ws.scan_state[k] = 0ull;
  __syncthreads();
  uint32_t wc_hits = 0;
  for (uint32_t b = blockIdx.x * PROBE_CHUNK; b < P; b += gridDim.x * PROBE_CHUNK) {
    uint32_t idx[PROBE_U], s0[PROBE_U], m[PROBE_U];
#pragma unroll
    for (uint32_t u = 0; u < PROBE_U; ++u) {
      idx[u] = b + u * PROBE_BLOCK + threadIdx.x;
      const bool in = idx[u] < P;
      s0[u] = in ? a.ws.piece_start[idx[u]] : 0u;
      m[u] = in ? a.ws.piece_start[idx[u] + 1] - s0[u] : 0u;
    }
    uint64_t spw[PROBE_U];
    UnitBytes<32> ub[PROBE_U];
#pragma unroll
    for (uint32_t u = 0; u < PROBE_U; ++u) {
      spw[u] = m[u] ? a.ws.spst[s0[u] >> 6] : 0ull;
      load_unit(a.text, a.n, s0[u], min(m[u], 32u), ub[u]);
    }
    // (a unit of two bytes is one key or two atoms: the pair table says
    // which; longer units probe the key table, whose second word holds key
    // bytes 8-15 and is read for units longer than 8 bytes only; the loads a
    // unit does not need go to entry 0, so that they cost no extra lines)
    uint64_t h[PROBE_U], k8[PROBE_U], k8b[PROBE_U];
    uint32_t slot[PROBE_U];
    Slot sl[PROBE_U];
    uint64_t ex[PROBE_U];
    int32_t pr[PROBE_U];
#pragma unroll
    for (uint32_t u = 0; u < PROBE_U; ++u) {
      const uint32_t len = min(max(m[u], 1u), 32u);
      unit_hash(ub[u], 0, len, h[u], k8[u], k8b[u]);
      slot[u] = m[u] > 2 ? uint32_t(h[u]) & T.slot_mask : 0u;
      sl[u] = T.slots[slot[u]];
      ex[u] = T.ext[m[u] > 8 ? slot[u] : 0u];
      pr[u] = T.pair[m[u] == 2 ? (ub[u].byte(0) << 8) | ub[u].byte(1) : 0u];
    }
    int cls[PROBE_U];
#pragma unroll
    for (uint32_t u = 0; u < PROBE_U; ++u) {
      cls[u] = -1;  // MergeList of a unit left to merge
      const uint32_t mm = m[u], s = s0[u];
      if (mm == 0) continue;
      int32_t id = -1;
      if ((spw[u] >> (s & 63)) & 1) {
        id = special_id(T, a.text + s, mm);
      } else if (mm == 1) {
        id = s_atom[ub[u].byte(0)];
      } else if (mm == 2) {
        if (pr[u] != RANK_NONE) {
          id = pr[u];
        } else {  // no merge: its two atoms, as the merge would write them
          a.ws.tmp_ids[s] = s_atom[ub[u].byte(0)];
          a.ws.tmp_ids[s + 1] = s_atom[ub[u].byte(1)];
          a.ws.piece_cnt[idx[u]] = 2u;
        }
      } else if (mm <= 32) {
        uint32_t meta = 0;
        const UnitBytes<32> &uu = ub[u];
        const int32_t r = mm <= T.max_key_len
                              ? probe_from(T, slot[u], sl[u], ex[u], k8[u], k8b[u], mm, meta,
                                           [&](const uint8_t *bb) __attribute__((always_inline)) { return unit_rest_eq(uu, 0, mm, bb); })
                              : RANK_NONE;
        if (r != RANK_NONE && (meta & META_SELF)) id = r;
        else cls[u] = mm <= 4 ? ML_4 : mm <= 8 ? ML_8 : mm <= 16 ? ML_16 : ML_32;
      } else {
        uint32_t meta = 0;
        const int32_t r = mm <= T.max_key_len ? lookup_text(T, a.text + s, mm, meta) : RANK_NONE;
        if (r != RANK_NONE && (meta & META_SELF)) id = r;
        else cls[u] = mm <= 128 ? ML_G128 : mm <= 256 ? ML_G256 : mm <= WAVE_MAX ? ML_G512 : ML_LONG;
      }
      a.ws.uid[idx[u]] = id >= 0 ? id : UID_MERGED;
      if (a.word_cache && cls[u] >= 0 && cls[u] <= int(ML_16))  // this unit under its hash
        a.ws.owner[owner_slot(h[u], a.owner_mask)] = idx[u];
    }
    if (WC) {
      // the kept word cache: the first 64 bytes of every unit's home entry
      // (its bytes, meta and first 7 ids) loaded together, then resolved;
      // a home entry holding other bytes sends the unit on to the next slots
      uint4 eq[PROBE_U][4];
      bool want[PROBE_U];
#pragma unroll
      for (uint32_t u = 0; u < PROBE_U; ++u) {
        want[u] = cls[u] >= 0 && cls[u] <= int(ML_32);
        const uint4 *e = reinterpret_cast<const uint4 *>(
            a.wcache + uint64_t(wc_slot(h[u], a.wc_mask)) * WC_WORDS);
#pragma unroll
        for (int q = 0; q < 4; ++q) eq[u][q] = want[u] ? e[q] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (uint32_t u = 0; u < PROBE_U; ++u) {
        if (!want[u]) continue;
        const uint32_t meta = eq[u][2].x, mm = m[u], s = s0[u];
        if (!(meta & WC_FULL)) continue;  // empty home slot: not cached
        const uint32_t k[8] = {eq[u][0].x, eq[u][0].y, eq[u][0].z, eq[u][0].w,
                               eq[u][1].x, eq[u][1].y, eq[u][1].z, eq[u][1].w};
        bool same = ((meta >> 8) & 63u) == mm;
#pragma unroll
        for (int q = 0; q < 8; ++q) same = same && k[q] == ub[u].d[q];
        bool hit = false;
        if (same) {
          const uint32_t cnt = meta & 63u;
          const uint32_t first[7] = {eq[u][2].y, eq[u][2].z, eq[u][2].w, eq[u][3].x,
                                     eq[u][3].y, eq[u][3].z, eq[u][3].w};
          const uint32_t *e = a.wcache + uint64_t(wc_slot(h[u], a.wc_mask)) * WC_WORDS;
#pragma unroll
          for (uint32_t j = 0; j < 7; ++j)
            if (j < cnt) a.ws.tmp_ids[s + j] = int32_t(first[j]);
          for (uint32_t j = 7; j < cnt; ++j) a.ws.tmp_ids[s + j] = int32_t(e[9 + j]);
          a.ws.piece_cnt[idx[u]] = cnt;
          hit = true;
        } else {
          hit = wc_find(a, ub[u], mm, h[u], s, idx[u], 1);
        }
        if (hit) {
          cls[u] = -1;  // settled from the kept word cache
          ++wc_hits;
        }
      }
    }
    if (threadIdx.x < ML_COUNT) {
      s_cnt[threadIdx.x] = 0;
      s_cur[threadIdx.x] = 0;
    }
    __syncthreads();
#pragma unroll
    for (uint32_t u = 0; u < PROBE_U; ++u)
      if (cls[u] >= 0) atomicAdd(&s_cnt[cls[u]], 1u);
    __syncthreads();
    if (threadIdx.x < ML_COUNT) {
      uint32_t o = 0;
      for (uint32_t L = 0; L < threadIdx.x; ++L) o += s_cnt[L];
      s_off[threadIdx.x] = o;
      if (s_cnt[threadIdx.x]) s_base[threadIdx.x] = atomicAdd(&st->n_list[threadIdx.x], s_cnt[threadIdx.x]);
    }
    __syncthreads();
#pragma unroll
    for (uint32_t u = 0; u < PROBE_U; ++u)
      if (cls[u] >= 0) s_list[s_off[cls[u]] + atomicAdd(&s_cur[cls[u]], 1u)] = idx[u];
    __syncthreads();
#pragma unroll
    for (uint32_t L = 0; L < ML_COUNT; ++L) {
      uint32_t *list = a.ws.lst[L];
      const uint32_t o = s_off[L];
      for (uint32_t k = threadIdx.x; k < s_cnt[L]; k += PROBE_BLOCK) list[s_base[L] + k] = s_list[o + k];
    }
    __syncthreads();
  }
  if (WC) {
    wc_hits = wave_sum(wc_hits);
    if ((threadIdx.x & 63) == 0 && wc_hits) atomicAdd(&st->wc_hits, (unsigned long long)wc_hits);
  }
}
__global__ void __launch_bounds__(PROBE_BLOCK) k_probe(EncodeArgs a) { probe_body<4, false>(a); }
__global__ void __launch_bounds__(PROBE_BLOCK) k_probe1(EncodeArgs a) { probe_body<1, false>(a); }
__global__ void __launch_bounds__(PROBE_BLOCK) k_probe2(EncodeArgs a) { probe_body<2, false>(a); }
// the same with the kept word cache
__global__ void __launch_bounds__(PROBE_BLOCK) k_probe_wc(EncodeArgs a) { probe_body<4, true>(a); }
__global__ void __launch_bounds__(PROBE_BLOCK) k_probe1_wc(EncodeArgs a) { probe_body<1, true>(a); }

// ---------------------------------------------------------------------------
// Group tier: units of 33..WAVE_MAX bytes, a group of G lanes per unit (64/G
// units per wave), P positions per lane in registers.  Position j of a unit
// lives in lane j % G of its group, slot j / G: its pair rank (RANK_NONE
// unless a part with a right neighbour starts at j) and the id of the part
// starting at j.  The part starts are a G-bit mask per slot, the same in
// every lane of the group.  Each round: group argmin (butterfly over the
// group's lanes, then the lowest position holding it), then two lanes of
// the group look up the merged part's new pairs side by side.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int32_t wave_min_i32(int32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const int32_t o = __shfl_xor(v, d, 64);
    v = o < v ? o : v;
  }
  return __builtin_amdgcn_readfirstlane(v);
}

// Minimum over the 64 lanes by DPP (row shifts, then row broadcasts 15 and
// 31; no LDS round trips), read back from lane 63.
__device__ __forceinline__ int32_t dpp_wave_min(int32_t v) {
  constexpr int32_t I = 0x7fffffff;
  v = min(v, __builtin_amdgcn_update_dpp(I, v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = min(v, __builtin_amdgcn_update_dpp(I, v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = min(v, __builtin_amdgcn_update_dpp(I, v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = min(v, __builtin_amdgcn_update_dpp(I, v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = min(v, __builtin_amdgcn_update_dpp(I, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = min(v, __builtin_amdgcn_update_dpp(I, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

template <uint32_t G, uint32_t P>
struct GroupMask {
  uint64_t w[P];
  static constexpr uint64_t full = G == 64 ? ~0ull : ((1ull << G) - 1);
  // first set position >= x, or m
  __device__ __forceinline__ uint32_t next(uint32_t x, uint32_t m) const {
    uint32_t res = m;
#pragma unroll
    for (int t = int(P) - 1; t >= 0; --t) {
      const uint32_t lo = G * uint32_t(t);
      uint64_t v = w[t];
      if (x >= lo + G) v = 0;
      else if (x > lo) v &= ~0ull << (x - lo);
      res = v ? lo + uint32_t(__ffsll(static_cast<unsigned long long>(v)) - 1) : res;
    }
    return res;
  }
  // last set position < x, or -1
  __device__ __forceinline__ int prev(uint32_t x) const {
    int res = -1;
#pragma unroll
    for (int t = 0; t < int(P); ++t) {
      const uint32_t lo = G * uint32_t(t);
      uint64_t v = w[t];
      if (x <= lo) v = 0;
      else if (x < lo + G) v &= (1ull << (x - lo)) - 1;
      res = v ? int(lo) + 63 - __clzll(static_cast<long long>(v)) : res;
    }
    return res;
  }
};

template <uint32_t G, uint32_t P>
__device__ void merge_group(const EncodeArgs &a, const uint32_t *list, uint32_t count,
                            uint32_t first, int lane) {
  const DevTables &T = a.T;
  const uint32_t g = uint32_t(lane) / G, gl = uint32_t(lane) % G;
  const uint32_t x = first + g;
  const bool live = x < count;
  const uint32_t i = live ? list[x] : 0u;
  const uint32_t s = live ? a.ws.piece_start[i] : 0u;
  const uint32_t m = live ? a.ws.piece_start[i + 1] - s : 0u;
  const uint8_t *p = a.text + s;
  int32_t r[P], pr[P];
  GroupMask<G, P> A;
#pragma unroll
  for (uint32_t t = 0; t < P; ++t) {
    const uint32_t j = G * t + gl;
    const uint32_t b0 = j < m ? p[j] : 0u, b1 = j + 1 < m ? p[j + 1] : 0u;
    r[t] = j + 1 < m ? T.pair[b0 * 256u + b1] : RANK_NONE;
    pr[t] = j < m ? T.atom[b0] : 0;
    const uint32_t lo = G * t;
    A.w[t] = m >= lo + G ? A.full : (m > lo ? (1ull << (m - lo)) - 1 : 0ull);
  }
  for (;;) {
    int32_t best = RANK_NONE;
#pragma unroll
    for (uint32_t t = 0; t < P; ++t) best = r[t] < best ? r[t] : best;
    if (G == 64) {
      best = dpp_wave_min(best);
    } else {
#pragma unroll
      for (uint32_t d = 1; d < G; d <<= 1) {
        const int32_t o = __shfl_xor(best, int(d), 64);
        best = o < best ? o : best;
      }
    }
    const bool act = best != RANK_NONE;
    if (!__ballot(act)) break;  // every group of the wave is done
    uint32_t bj = m;  // lowest position of the group holding the minimum
#pragma unroll
    for (int t = int(P) - 1; t >= 0; --t) {
      const unsigned long long bal = __ballot(act && r[t] == best);
      const uint64_t gb = (bal >> (g * G)) & A.full;
      bj = gb ? G * uint32_t(t) + uint32_t(__ffsll(static_cast<unsigned long long>(gb)) - 1) : bj;
    }
    uint32_t k = m, k2 = m;
    int q = -1;
    if (act) {
      k = A.next(bj + 1, m);   // the part merged into bj
      k2 = A.next(k + 1, m);   // end of the merged part
      q = A.prev(bj);
    }
    // ids of the parts starting at k2 and q, read from the lanes holding them
    const uint32_t uq = uint32_t(q);
    int32_t v2 = 0, vq = 0;
#pragma unroll
    for (uint32_t t = 0; t < P; ++t) {
      v2 = k2 / G == t ? pr[t] : v2;
      vq = uq / G == t ? pr[t] : vq;
    }
    const int32_t id2 = __shfl(v2, int(g * G + k2 % G), 64);
    const int32_t idq = __shfl(vq, int(g * G + uq % G), 64);
    // group lane 0: the merged part (id best) with its right neighbour; lane
    // 1: the left neighbour with the merged part
    int32_t rv = RANK_NONE;
    if (act && gl == 0 && k2 < m) rv = merge_rank(T, uint32_t(best), uint32_t(id2));
    if (act && gl == 1 && q >= 0) rv = merge_rank(T, uint32_t(idq), uint32_t(best));
    const int32_t nb = __shfl(rv, int(g * G), 64), nq = __shfl(rv, int(g * G + 1), 64);
    if (act) {
#pragma unroll
      for (uint32_t t = 0; t < P; ++t) {
        const uint32_t j = G * t + gl;
        r[t] = j == k ? RANK_NONE : r[t];
        r[t] = j == bj ? nb : r[t];
        pr[t] = j == bj ? best : pr[t];
        r[t] = (q >= 0 && j == uint32_t(q)) ? nq : r[t];
        A.w[t] = (k / G) == t ? A.w[t] & ~(1ull << (k % G)) : A.w[t];
      }
    }
  }
  if (!live) return;
  uint32_t c = 0;
  const uint64_t below = (1ull << gl) - 1;
#pragma unroll
  for (uint32_t t = 0; t < P; ++t) {
    if ((A.w[t] >> gl) & 1) a.ws.tmp_ids[s + c + uint32_t(__popcll(A.w[t] & below))] = pr[t];
    c += uint32_t(__popcll(A.w[t]));
  }
  a.ws.piece_cnt[i] = c;  // c is the same in every lane of the group
}

// ---------------------------------------------------------------------------
// Long tier: one workgroup per unit longer than WAVE_MAX.  Per position j of
// the unit (text byte s + j): lrank = rank of the pair that starts with the
// part starting at j, in global memory; lpart = id of that part, in LDS for
// units of up to LONG_LDS_POS bytes, else in global memory.  Per 64-position
// block b of the unit: part starts, pairs chosen this round, the part starts
// whose pair has the block's least rank, that least rank, least rank stale;
// in LDS for units of up to 64 * LONG_LDS_BLOCKS bytes, else in global
// memory at index (s >> 5) + b (a unit of m > 64 bytes needs ceil(m/64) <=
// floor(m/32) entries, so units never share one): lbits, lsel, leqm, lmin,
// ldirty.  (gfx950 gives one workgroup up to 160 KB of LDS.)
//
// Each round takes the least rank R and merges in one batch the leftmost
// non-overlapping pairs of rank R: in every run of consecutive parts whose
// pairs all rank R, the 1st, 3rd, 5th ... pair.  Taken one at a time in text
// order these are exactly the merges the one-at-a-time loop makes, as long as
// every pair it creates on the way ranks above R; so the two pairs each merge
// creates are looked up in the state the one-at-a-time loop has at that merge
// (the part before it already merged if it was chosen, the part after it not
// yet), and the batch stops after the first merge that creates a pair of rank
// <= R.  The leftmost pair of rank R is always chosen, so every round merges.
// Runs of one repeated character (tens of thousands of spaces) take a few
// rounds per doubling of the part length instead of one round per merge.
// Threads own blocks (or quarter blocks); barriers order the phases of a round.
// ---------------------------------------------------------------------------
struct LongUnit {
  const EncodeArgs &a;
  uint32_t s, m, nb;
  unsigned long long *bits, *sel, *eqm;
  int32_t *mn;
  uint32_t *dirty;
  int32_t *pt;  // part ids, position 0 of the unit
  __device__ __forceinline__ int32_t &rank(uint32_t j) const { return a.ws.lrank[s + j]; }
  __device__ __forceinline__ int32_t &part(uint32_t j) const { return pt[j]; }
  // first part start >= x, or m
  __device__ __forceinline__ uint32_t next(uint32_t x) const {
    if (x >= m) return m;
    uint32_t b = x >> 6;
    unsigned long long w = bits[b] & (~0ull << (x & 63));
    while (!w) {
      if (++b >= nb) return m;
      w = bits[b];
    }
    return min(m, 64 * b + uint32_t(__ffsll(w) - 1));
  }
  // last part start < x, or -1
  __device__ __forceinline__ int prev(uint32_t x) const {
    if (x == 0) return -1;
    const uint32_t y = x - 1;
    uint32_t b = y >> 6;
    unsigned long long w = bits[b] & ((y & 63) == 63 ? ~0ull : ((2ull << (y & 63)) - 1));
    while (!w) {
      if (b == 0) return -1;
      w = bits[--b];
    }
    return int(64 * b + 63 - uint32_t(__clzll(static_cast<long long>(w))));
  }
  __device__ __forceinline__ bool chosen(uint32_t j) const { return (sel[j >> 6] >> (j & 63)) & 1; }
  // Pair ranks of the part starts of block b: the least one, and the mask of
  // the starts whose pair has it (empty when no pair has a rank).  All 64
  // loads are issued without branches (addresses clamped into the unit) so
  // that they overlap.
  __device__ __forceinline__ int32_t block_scan(uint32_t b, unsigned long long A,
                                                unsigned long long &eq) const {
    int32_t r = RANK_NONE;
    eq = 0;
    const uint32_t j0 = 64 * b;
#pragma unroll
    for (uint32_t q = 0; q < 64; q += 8) {
      int32_t v[8];
#pragma unroll
      for (uint32_t t = 0; t < 8; ++t) v[t] = rank(min(j0 + q + t, m - 1));
#pragma unroll
      for (uint32_t t = 0; t < 8; ++t) {
        const int32_t x = ((A >> (q + t)) & 1) ? v[t] : RANK_NONE;
        eq = x < r ? (1ull << (q + t)) : (x == r ? eq | (1ull << (q + t)) : eq);
        r = min(r, x);
      }
    }
    return r == RANK_NONE ? (eq = 0, r) : r;
  }
  __device__ __forceinline__ void rescan(uint32_t b) const {
    unsigned long long e;
    mn[b] = block_scan(b, bits[b], e);
    eqm[b] = e;
  }
};

// Chain-parity function of a block: bit 1 = constant, bit 0 = value (xor
// mask if not constant).  State = "the next pair of rank R in the current
// run of such pairs has an odd index".
__device__ __forceinline__ uint32_t chain_then(uint32_t f, uint32_t g) {
  if (g & 2) return g;
  return (f & 2) | ((f ^ g) & 1);
}

template <int SK, bool WC>
__device__ __forceinline__ void merge_short_unit(const EncodeArgs &a, const int32_t *atom, uint32_t i,
                                                 const PartCol &lp) {
  const uint32_t s = a.ws.piece_start[i];
  const uint32_t m = a.ws.piece_start[i + 1] - s;
  UnitBytes<SK> u;
  load_unit(a.text, a.n, s, m, u);
  const uint32_t cnt = merge_short<SK>(a.T, atom, u, m, lp, a.ws.tmp_ids + s);
  a.ws.piece_cnt[i] = cnt;
  if (WC) wc_put(a, u, m, s, cnt);
}

// Short-tier work item with the word cache: list entries first .. first +
// 64 K - 1 of one class of 2-16 bytes, K per lane.  The election of all K
// entries runs with their loads issued side by side (the entries, their
// offsets and bytes, their slots, the slot units' offsets and bytes); a unit
// that follows another records it (uid) and is done; the leaders are packed
// into a queue in LDS and merged 64 at a time, one lane each.
template <int SK, uint32_t K, bool ELECT, bool WC>
__device__ __forceinline__ void merge_short_item(const EncodeArgs &a, uint32_t P, const int32_t *atom,
                                                 const PartCol &lp, uint32_t *queue,
                                                 const uint32_t *list, uint32_t count,
                                                 uint32_t first, int lane) {
  if (!ELECT) {  // every entry merges itself, one lane each
#pragma unroll
    for (uint32_t k = 0; k < K; ++k) {
      const uint32_t x = first + 64 * k + uint32_t(lane);
      if (x < count) merge_short_unit<SK, WC>(a, atom, list[x], lp);
    }
    return;
  }
  uint32_t idx[K], s0[K], m[K], own[K], js[K], jm[K];
  bool in[K], other[K];
  UnitBytes<SK> u[K], v[K];
#pragma unroll
  for (uint32_t k = 0; k < K; ++k) {
    const uint32_t x = first + 64 * k + uint32_t(lane);
    in[k] = x < count;
    idx[k] = in[k] ? list[x] : 0u;
  }
#pragma unroll
  for (uint32_t k = 0; k < K; ++k) {
    s0[k] = in[k] ? a.ws.piece_start[idx[k]] : 0u;
    m[k] = in[k] ? a.ws.piece_start[idx[k] + 1] - s0[k] : 0u;
  }
#pragma unroll
  for (uint32_t k = 0; k < K; ++k) load_unit(a.text, a.n, s0[k], m[k], u[k]);
#pragma unroll
  for (uint32_t k = 0; k < K; ++k) {
    uint64_t h, k8, k8b;
    unit_hash(u[k], 0, max(m[k], 1u), h, k8, k8b);
    own[k] = in[k] ? a.ws.owner[owner_slot(h, a.owner_mask)] : 0u;
  }
#pragma unroll
  for (uint32_t k = 0; k < K; ++k) {
    other[k] = in[k] && own[k] != idx[k] && own[k] < P && own[k] <= FOLLOW_MAX;
    js[k] = other[k] ? a.ws.piece_start[own[k]] : 0u;
    jm[k] = other[k] ? a.ws.piece_start[own[k] + 1] - js[k] : 0u;
  }
#pragma unroll
  for (uint32_t k = 0; k < K; ++k) {
    other[k] = other[k] && jm[k] == m[k];
    load_unit(a.text, a.n, js[k], other[k] ? m[k] : 0u, v[k]);
  }
  uint32_t nq = 0;  // leaders queued (the same in every lane)
#pragma unroll
  for (uint32_t k = 0; k < K; ++k) {
    const bool follow = other[k] && v[k] == u[k];
    if (follow) a.ws.uid[idx[k]] = UID_FOLLOW - int32_t(own[k]);
    const bool lead = in[k] && !follow;
    const unsigned long long b = __ballot(lead);
    if (lead) queue[nq + uint32_t(__popcll(b & ((1ull << lane) - 1)))] = idx[k];
    nq += uint32_t(__popcll(b));
  }
  __syncthreads();  // (one wave: orders the queue's writes before its reads)
  for (uint32_t q = 0; q < nq; q += 64) {
    const uint32_t x = q + uint32_t(lane);
    if (x < nq) merge_short_unit<SK, WC>(a, atom, queue[x], lp);
  }
  __syncthreads();  // the queue is rewritten by the next item
}

// Merge of the units of 2-16 bytes: work items of list entries of one
// length class (256 with the word cache, else 64), longest class first; the register
// tiers follow the class, so that a wave's rounds and its per-round work
// follow its longest unit.  Wave w takes items w, w + G, w + 2G, ... (G
// waves in the grid).  The item index is wave-uniform by construction: no
// lane-0 ticket and broadcast, which lets the compiler split the loop per
// lane.
constexpr uint32_t SHORT_K = 4;  // chunks of 64 entries per item
// (ELECT: the per-call word cache, texts from WORD_CACHE_MIN bytes.  The LDS
// of a wave -- atoms, part ids of up to 16 positions per lane, the leaders'
// queue only with the cache -- sets how many merge waves share a CU.
// FEW32: up to FEW32_MAX units of 17-32 bytes are taken here too, 32 lanes
// each with one position per lane, as the first items, so that their long
// chains start first; k_merge_wide then leaves them out.)
template <bool WC, bool ELECT, bool FEW32>
__device__ __forceinline__ void merge_body(const EncodeArgs &a) {
  if (a.ws.status->pad2) return;
  const Status *st = a.ws.status;
  const int lane = int(threadIdx.x);
  const uint32_t P = uint32_t(st->n_pieces);
  const uint32_t n16 = st->n_list[ML_16], n8 = st->n_list[ML_8], n4 = st->n_list[ML_4];
  const uint32_t n32 = st->n_list[ML_32];
  const uint32_t f32 = (FEW32 && n32 <= FEW32_MAX) ? (n32 + 1) / 2 : 0u;
  // entries per item: 256 with the word cache (elected together), else 64
  const uint32_t C = ELECT ? 64 * SHORT_K : 64;
  const uint32_t e16 = f32 + (n16 + C - 1) / C, e8 = e16 + (n8 + C - 1) / C, e4 = e8 + (n4 + C - 1) / C;
  if (blockIdx.x >= e4) return;
  __shared__ int32_t s_atom[256];
  __shared__ uint16_t s_part_lo[16 * 64];  // [position][lane]: part ids of each lane's unit
  __shared__ uint8_t s_part_hi[16 * 64];
  __shared__ uint32_t s_queue[ELECT ? 64 * SHORT_K : 1];
  const PartCol lp{s_part_lo + lane, s_part_hi + lane};
  reinterpret_cast<int4 *>(s_atom)[lane] = reinterpret_cast<const int4 *>(a.T.atom)[lane];
  __syncthreads();
  for (uint32_t item = blockIdx.x; item < e4; item += gridDim.x) {
    if (FEW32 && item < f32) {
      merge_group<32, 1>(a, a.ws.lst[ML_32], n32, item * 2, lane);
      continue;
    }
    const bool in16 = item < e16, in8 = !in16 && item < e8;
    const uint32_t first = (item - (in16 ? f32 : in8 ? e16 : e8)) * C;
    if constexpr (ELECT) {
      if (in16)
        merge_short_item<16, SHORT_K, true, WC>(a, P, s_atom, lp, s_queue, a.ws.lst[ML_16], n16, first, lane);
      else if (in8)
        merge_short_item<8, SHORT_K, true, WC>(a, P, s_atom, lp, s_queue, a.ws.lst[ML_8], n8, first, lane);
      else
        merge_short_item<4, SHORT_K, true, WC>(a, P, s_atom, lp, s_queue, a.ws.lst[ML_4], n4, first, lane);
    } else {
      if (in16)
        merge_short_item<16, 1, false, WC>(a, P, s_atom, lp, s_queue, a.ws.lst[ML_16], n16, first, lane);
      else if (in8)
        merge_short_item<8, 1, false, WC>(a, P, s_atom, lp, s_queue, a.ws.lst[ML_8], n8, first, lane);
      else
        merge_short_item<4, 1, false, WC>(a, P, s_atom, lp, s_queue, a.ws.lst[ML_4], n4, first, lane);
    }
  }
}
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) k_merge(EncodeArgs a) {
  merge_body<false, false, true>(a);
}
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) k_merge_elect(EncodeArgs a) {
  merge_body<false, true, false>(a);
}
// the same with the kept word cache
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) k_merge_wc(EncodeArgs a) {
  merge_body<true, false, false>(a);
}
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) k_merge_elect_wc(EncodeArgs a) {
  merge_body<true, true, false>(a);
}

// Merge of the units of 17..WAVE_MAX bytes (second stream, beside k_merge:
// theirs are the longest chains of dependent merge rounds below the long
// tier, and running them apart lets them start with the rest), longest
// first.  Units of 33..WAVE_MAX bytes: few, one wave each, positions per
// lane sized to the list's longest unit (their chains are the critical
// path, and a wave shared by several units waits for the slowest probe of
// all of them every round); many, 16 or 32 lanes per unit, for throughput.
// Then the units of 17-32 bytes, one lane each, 64 per item (nearly every
// such unit is a byte string of its own, so they skip the word cache).
template <bool WC, bool FEW32>
__device__ __forceinline__ void merge_wide_body(const EncodeArgs &a) {
  if (a.ws.status->pad2) return;
  const Status *st = a.ws.status;
  const int lane = int(threadIdx.x);
  const uint32_t n64 = st->n_list[ML_G512], n32g = st->n_list[ML_G256], n16g = st->n_list[ML_G128];
  const uint32_t n32 = st->n_list[ML_32];
  const bool pack = n64 + n32g + n16g > GROUP_PACK_MIN;
  const uint32_t e64 = n64, e32g = e64 + (pack ? (n32g + 1) / 2 : n32g);
  const uint32_t e16g = e32g + (pack ? (n16g + 3) / 4 : n16g);
  // (FEW32: up to FEW32_MAX units of 17-32 bytes are k_merge's; else they
  // are taken here, one lane each, positions in registers)
  const bool few32 = FEW32 && n32 <= FEW32_MAX;
  const uint32_t e32 = e16g + (few32 ? 0u : (n32 + 63) / 64);
  if (blockIdx.x >= e32) return;
  __shared__ int32_t s_atom[256];
  __shared__ uint16_t s_part_lo[32 * 64];  // [position][lane]: part ids of each lane's unit
  __shared__ uint8_t s_part_hi[32 * 64];
  const PartCol lp{s_part_lo + lane, s_part_hi + lane};
  reinterpret_cast<int4 *>(s_atom)[lane] = reinterpret_cast<const int4 *>(a.T.atom)[lane];
  __syncthreads();
  for (uint32_t item = blockIdx.x; item < e32; item += gridDim.x) {
    if (item < e64) {
      merge_group<64, 8>(a, a.ws.lst[ML_G512], n64, item, lane);
    } else if (item < e32g) {
      if (pack) merge_group<32, 8>(a, a.ws.lst[ML_G256], n32g, (item - e64) * 2, lane);
      else merge_group<64, 4>(a, a.ws.lst[ML_G256], n32g, item - e64, lane);
    } else if (item < e16g) {
      if (pack) merge_group<16, 8>(a, a.ws.lst[ML_G128], n16g, (item - e32g) * 4, lane);
      else merge_group<64, 2>(a, a.ws.lst[ML_G128], n16g, item - e32g, lane);
    } else {
      const uint32_t x = (item - e16g) * 64 + uint32_t(lane);
      if (x < n32) merge_short_unit<32, WC>(a, s_atom, a.ws.lst[ML_32][x], lp);
    }
  }
}
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) k_merge_wide(EncodeArgs a) {
  merge_wide_body<false, false>(a);
}
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) k_merge_wide_few32(EncodeArgs a) {
  merge_wide_body<false, true>(a);
}
// the same with the kept word cache
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) k_merge_wide_wc(EncodeArgs a) {
  merge_wide_body<true, false>(a);
}

// Block-wide helpers of the long tier (LONG_BLOCK threads, LDS scratch sh).
constexpr uint32_t LONG_BLOCK = 1024;

__device__ __forceinline__ int32_t block_min_i32(int32_t v, int32_t *sh) {
  v = wave_min_i32(v);
  const uint32_t wv = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) sh[wv] = v;
  __syncthreads();
  int32_t r = RANK_NONE;
#pragma unroll
  for (uint32_t k = 0; k < LONG_BLOCK / 64; ++k) r = min(r, sh[k]);
  __syncthreads();
  return r;
}

// inclusive scan of chain-parity functions over the threads, in thread order:
// wave scans by shuffles, then each wave folds in the totals of the waves
// before it (0 is the identity)
__device__ __forceinline__ uint32_t block_chain_scan(uint32_t f, uint32_t *sh) {
  const int lane = int(threadIdx.x & 63);
  const uint32_t wv = threadIdx.x / 64;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(f, d, 64);
    if (lane >= d) f = chain_then(o, f);
  }
  if (lane == 63) sh[wv] = f;
  __syncthreads();
  uint32_t pre = 0;
  for (uint32_t q = 0; q < wv; ++q) pre = chain_then(pre, sh[q]);
  __syncthreads();
  return chain_then(pre, f);
}

// exclusive sum over the threads; total to every thread
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t v, uint32_t *sh, uint32_t &total) {
  const uint32_t t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (uint32_t d = 1; d < LONG_BLOCK; d <<= 1) {
    const uint32_t o = t >= d ? sh[t - d] : 0u;
    __syncthreads();
    sh[t] += o;
    __syncthreads();
  }
  total = sh[LONG_BLOCK - 1];
  const uint32_t r = sh[t] - v;
  __syncthreads();
  return r;
}

// One workgroup per unit.  Blocks of 64 positions are owned by threads for
// the scans; the chosen pairs of a round are handled per quarter block (16
// positions), so that up to 4 * blocks threads merge side by side.
constexpr uint32_t LONG_LDS_BLOCKS = 512, LONG_LDS_POS = 25600;
struct LongLds {
  unsigned long long bits[LONG_LDS_BLOCKS], sel[LONG_LDS_BLOCKS], eqm[LONG_LDS_BLOCKS];
  int32_t mn[LONG_LDS_BLOCKS];
  uint32_t dirty[LONG_LDS_BLOCKS];
  int32_t part[LONG_LDS_POS];
};

// Units made of at most RLE_RUNS runs of one repeated byte (long runs of
// spaces, dashes, '=' ...) are merged in run-length form, one run of equal
// part ids (id, count) per lane of the first wave.  The pairs inside a run
// all have the rank of (id, id); the pair between two runs is one of a
// kind.  Each step takes the least rank R and the leftmost pair that has
// it, as the one-at-a-time loop does.  A pair between two runs merges
// alone: (x, c), (y, d) become (x, c - 1), (R, 1), (y, d - 1).  A pair
// inside a run (x, c) starts a batch: the loop merges the run's parts two
// by two, left to right, into parts R for as long as every pair these
// merges create ranks above R (the first creates (left neighbour, R) and
// (R, x), later ones (R, R) and again (R, x)); once one ranks at or below R
// the loop takes it next, so the batch stops after the first merge, or the
// second, or runs through the whole run: (x, c) becomes (R, k),
// (x, c - 2k).  Runs with equal neighbours are joined.  Returns false, with
// nothing written, when the runs do not fit in a wave or the steps exceed
// RLE_STEPS; the unit is then merged position by position.  (Merging a run
// of n equal bytes takes a few steps per doubling of the part length.)
constexpr uint32_t RLE_RUNS = 64, RLE_STEPS = 4096;

__device__ bool merge_long_runs(const EncodeArgs &a, uint32_t i, uint32_t s, uint32_t m,
                                int32_t *scratch) {
  const DevTables &T = a.T;
  const uint32_t tid = threadIdx.x;
  const uint8_t *p = a.text + s;
  // runs of equal bytes: their starts, in no order, at most RLE_RUNS of them
  // kept (positions tid, tid + LONG_BLOCK, ..., eight loads in flight)
  uint32_t *nst = reinterpret_cast<uint32_t *>(scratch + 4 * RLE_RUNS);
  if (tid == 0) *nst = 0u;
  __syncthreads();
  for (uint32_t k0 = 0; k0 * LONG_BLOCK < m; k0 += 8) {
    uint32_t b[8], pb[8];
#pragma unroll
    for (uint32_t q = 0; q < 8; ++q) {
      const uint32_t j = tid + (k0 + q) * LONG_BLOCK;
      b[q] = j < m ? uint32_t(p[j]) : 0u;
      pb[q] = (j < m && j > 0) ? uint32_t(p[j - 1]) : 0x100u;
    }
#pragma unroll
    for (uint32_t q = 0; q < 8; ++q) {
      const uint32_t j = tid + (k0 + q) * LONG_BLOCK;
      if (j < m && b[q] != pb[q]) {
        const uint32_t o = atomicAdd(nst, 1u);
        if (o < RLE_RUNS) scratch[o] = int32_t(j);
      }
    }
  }
  __syncthreads();
  const uint32_t nruns = *nst;
  if (nruns > RLE_RUNS) return false;
  int32_t *fid = scratch + RLE_RUNS;
  uint32_t *fcnt = reinterpret_cast<uint32_t *>(scratch + 2 * RLE_RUNS);
  uint32_t *fres = reinterpret_cast<uint32_t *>(scratch + 3 * RLE_RUNS);  // [runs, ok]
  if (tid < 64) {
    const int lane = int(tid);
    int nr = int(nruns);
    // the starts in text order: lane l sends its start to the lane of its
    // rank among them
    const int32_t v = lane < nr ? scratch[lane] : 0x7FFFFFFF;
    int rk = 0;
    for (int q = 0; q < nr; ++q) rk += __shfl(v, q, 64) < v ? 1 : 0;
    const int32_t st_sorted = __builtin_amdgcn_ds_permute((lane < nr ? rk : lane) * 4, v);
    const int32_t en_sorted = __shfl(st_sorted, min(lane + 1, 63), 64);
    int32_t id = 0, ra = RANK_NONE, rb = RANK_NONE;
    uint32_t cnt = 0;
    if (lane < nr) {
      const uint32_t st = uint32_t(st_sorted);
      const uint32_t en = lane + 1 < nr ? uint32_t(en_sorted) : m;
      const uint32_t b = p[st];
      const uint32_t nb = lane + 1 < nr ? uint32_t(p[en]) : 0u;
      id = T.atom[b];
      cnt = en - st;
      ra = T.pair[b * 256u + b];
      rb = lane + 1 < nr ? T.pair[b * 256u + nb] : RANK_NONE;
    }
    bool ok = true;
    for (uint32_t step = 0;; ++step) {  // wave-uniform
      const bool live = lane < nr;
      const int32_t va = (live && cnt >= 2) ? ra : RANK_NONE;
      const int32_t vb = (live && lane + 1 < nr) ? rb : RANK_NONE;
      const int32_t R = wave_min_i32(min(va, vb));
      if (R == RANK_NONE) break;
      if (step >= RLE_STEPS) {
        ok = false;
        break;
      }
      const unsigned long long ba = __ballot(va == R), bb = __ballot(vb == R);
      const int L = __ffsll(ba | bb) - 1;
      const bool inner = (ba >> L) & 1;
      const int32_t idL = __shfl(id, L, 64), idL1 = __shfl(id, min(L + 1, 63), 64);
      const int32_t idLm = __shfl(id, max(L - 1, 0), 64);
      const uint32_t cL = __shfl(cnt, L, 64), cL1 = __shfl(cnt, min(L + 1, 63), 64);
      // the runs that replace run L (inner) or runs L and L+1 (between)
      int32_t nid0, nid1, nid2;
      uint32_t nc0, nc1, nc2;
      int consumed;
      if (inner) {
        int32_t look = RANK_NONE;
        if (lane == 0 && L > 0) look = merge_rank(T, uint32_t(idLm), uint32_t(R));
        if (lane == 1 && cL >= 3) look = merge_rank(T, uint32_t(R), uint32_t(idL));
        if (lane == 2 && cL >= 4) look = merge_rank(T, uint32_t(R), uint32_t(R));
        const int32_t nl = __shfl(look, 0, 64), nx = __shfl(look, 1, 64), pp = __shfl(look, 2, 64);
        uint32_t k;
        if (cL < 4 || (L > 0 && nl <= R) || nx <= R) k = 1;
        else if (pp <= R) k = 2;
        else k = cL / 2;
        nid0 = R, nc0 = k;
        nid1 = idL, nc1 = cL - 2 * k;
        nid2 = 0, nc2 = 0;
        consumed = 1;
      } else {
        nid0 = idL, nc0 = cL - 1;
        nid1 = R, nc1 = 1;
        nid2 = idL1, nc2 = cL1 - 1;
        consumed = 2;
      }
      // the non-empty ones of the three, in order: e0, e1, e2
      const bool h0 = nc0 != 0, h1 = nc1 != 0, h2 = nc2 != 0;
      const int nn = int(h0) + int(h1) + int(h2);
      const int e0 = h0 ? 0 : (h1 ? 1 : 2), e1 = (h0 && h1) ? 1 : 2;
      const int shift = nn - consumed;
      if (nr + shift > int(RLE_RUNS)) {
        ok = false;
        break;
      }
      // lanes before L keep their run, L .. L+nn-1 take the new runs, the
      // rest take the run `shift` lanes before them
      const int src = min(max(lane - shift, 0), 63);
      const int32_t sid = __shfl(id, src, 64);
      const uint32_t scnt = __shfl(cnt, src, 64);
      if (lane >= L) {
        if (lane < L + nn) {
          const int t = lane - L;
          const int e = t == 0 ? e0 : (t == 1 ? e1 : 2);
          id = e == 0 ? nid0 : (e == 1 ? nid1 : nid2);
          cnt = e == 0 ? nc0 : (e == 1 ? nc1 : nc2);
        } else {
          id = sid;
          cnt = scnt;
        }
      }
      nr += shift;
      // join runs with equal neighbours
      for (;;) {
        const int32_t pid = __shfl_up(id, 1, 64);
        const unsigned long long eq = __ballot(lane > 0 && lane < nr && id == pid);
        if (!eq) break;
        const int f = __ffsll(eq) - 1;
        const uint32_t cf = __shfl(cnt, f, 64);
        if (lane == f - 1) cnt += cf;
        const int32_t nid = __shfl(id, min(lane + 1, 63), 64);
        const uint32_t ncnt = __shfl(cnt, min(lane + 1, 63), 64);
        if (lane >= f) {
          id = nid;
          cnt = ncnt;
        }
        --nr;
      }
      // ranks of every run: inside it and with the next run
      const int32_t nxt = __shfl(id, min(lane + 1, 63), 64);
      merge_rank2(T, lane < nr, uint32_t(id), uint32_t(id), lane + 1 < nr, uint32_t(id), uint32_t(nxt), ra, rb);
      if (lane >= nr) ra = RANK_NONE;
      if (lane + 1 >= nr) rb = RANK_NONE;
    }
    if (lane < nr) {
      fid[lane] = id;
      fcnt[lane] = cnt;
    }
    if (lane == 0) {
      fres[0] = uint32_t(nr);
      fres[1] = ok ? 1u : 0u;
    }
  }
  __syncthreads();
  const uint32_t nr = fres[0];
  const bool ok = fres[1] != 0;
  if (ok) {
    uint32_t o = 0;
    for (uint32_t r = 0; r < nr; ++r) {
      const uint32_t cr = fcnt[r];
      const int32_t ir = fid[r];
      for (uint32_t x = tid; x < cr; x += LONG_BLOCK) a.ws.tmp_ids[s + o + x] = ir;
      o += cr;
    }
    if (tid == 0) a.ws.piece_cnt[i] = o;
  }
  __syncthreads();
  return ok;
}

__device__ void merge_long(const EncodeArgs &a, uint32_t i, uint32_t *sh, LongLds &ld) {
  const DevTables &T = a.T;
  const uint32_t tid = threadIdx.x;
  const uint32_t s = a.ws.piece_start[i];
  const uint32_t m = a.ws.piece_start[i + 1] - s;
  const uint8_t *p = a.text + s;
  if (merge_long_runs(a, i, s, m, ld.part)) return;
  const uint32_t base = s >> 5;
  const uint32_t nbk = (m + 63) / 64;
  const bool in_lds = nbk <= LONG_LDS_BLOCKS;
  LongUnit U{a, s, m, nbk, in_lds ? ld.bits : a.ws.lbits + base, in_lds ? ld.sel : a.ws.lsel + base,
             in_lds ? ld.eqm : a.ws.leqm + base, in_lds ? ld.mn : a.ws.lmin + base,
             in_lds ? ld.dirty : a.ws.ldirty + base, m <= LONG_LDS_POS ? ld.part : a.ws.lpart + s};
  const uint32_t nb = U.nb;
  // initial pair ranks and atoms, eight positions per thread with their
  // loads issued before the stores
  for (uint32_t j0 = tid; j0 < m; j0 += 8 * LONG_BLOCK) {
    uint32_t c0[8], c1[8];
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) {
      const uint32_t j = j0 + k * LONG_BLOCK;
      c0[k] = j < m ? p[j] : 0u;
      c1[k] = j + 1 < m ? p[j + 1] : 0u;
    }
    int32_t rk[8], at[8];
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) {
      const uint32_t j = j0 + k * LONG_BLOCK;
      rk[k] = (j + 1 < m) ? T.pair[c0[k] * 256u + c1[k]] : RANK_NONE;
      at[k] = T.atom[c0[k]];
    }
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) {
      const uint32_t j = j0 + k * LONG_BLOCK;
      if (j < m) {
        U.rank(j) = rk[k];
        U.part(j) = at[k];
      }
    }
  }
  for (uint32_t b = tid; b < nb; b += LONG_BLOCK) {
    const uint32_t left = m - 64 * b;
    U.bits[b] = left >= 64 ? ~0ull : ((1ull << left) - 1);
    U.sel[b] = 0;
    U.dirty[b] = 0;
  }
  __syncthreads();
  for (uint32_t b = tid; b < nb; b += LONG_BLOCK) U.rescan(b);
  __syncthreads();

  for (;;) {
    int32_t R = RANK_NONE;
    for (uint32_t b = tid; b < nb; b += LONG_BLOCK) R = min(R, U.mn[b]);
    R = block_min_i32(R, reinterpret_cast<int32_t *>(sh));
    if (R == RANK_NONE) break;

    // 1. choose the pairs: chain parity scanned over blocks, LONG_BLOCK at a time
    uint32_t carry = 0;
    for (uint32_t b0 = 0; b0 < nb; b0 += LONG_BLOCK) {
      const uint32_t b = b0 + tid;
      unsigned long long A = 0, C = 0;
      if (b < nb) {
        A = U.bits[b];
        if (U.mn[b] == R) C = U.eqm[b];
      }
      const unsigned long long N = A & ~C;
      uint32_t f;
      if (A == 0) {
        f = 0;
      } else if (N == 0) {
        f = uint32_t(__popcll(C)) & 1u;
      } else {
        const int h = 63 - __clzll(static_cast<long long>(N));
        const unsigned long long after = h == 63 ? 0ull : (C & (~0ull << (h + 1)));
        f = 2u | (uint32_t(__popcll(after)) & 1u);
      }
      const uint32_t inc = block_chain_scan(f, sh);
      sh[tid] = inc;
      __syncthreads();
      const uint32_t ex = tid ? sh[tid - 1] : 0u;  // 0 = identity
      const uint32_t last = sh[LONG_BLOCK - 1];
      __syncthreads();
      uint32_t st = (ex & 2) ? (ex & 1) : (carry ^ (ex & 1));
      unsigned long long S = 0;
      unsigned long long w = A;
      while (w) {
        const uint32_t t = uint32_t(__ffsll(w) - 1);
        w &= w - 1;
        if ((C >> t) & 1) {
          if (st == 0) S |= 1ull << t;
          st ^= 1u;
        } else {
          st = 0;
        }
      }
      if (b < nb) U.sel[b] = S;
      carry = (last & 2) ? (last & 1) : (carry ^ (last & 1));
    }
    __syncthreads();

    // 2. the pairs each chosen merge creates, and the first merge after which
    // the batch must stop
    uint32_t stop = 0xFFFFFFFFu;
    // (thread x takes positions 2x and 2x+1, at most one of which begins a
    // chosen pair, so that neighbouring lanes touch neighbouring positions)
    for (uint32_t x = tid; x < 32 * nb; x += LONG_BLOCK) {
      const uint32_t b = x >> 5;
      const uint32_t two = uint32_t(U.sel[b] >> (2 * (x & 31))) & 3u;
      if (two) {
        const uint32_t j = 64 * b + 2 * (x & 31) + ((two & 1) ? 0u : 1u);
        const uint32_t k = U.next(j + 1);
        const uint32_t k2 = U.next(k + 1);
        const int y = U.prev(j);
        int pf = y;
        if (y >= 0) {
          const int z = U.prev(uint32_t(y));
          if (z >= 0 && U.chosen(uint32_t(z))) pf = z;  // y merged into z
        }
        // the merged part (id R) with its neighbours; a left neighbour that
        // merges in this batch too has id R as well
        const uint32_t lid = pf >= 0 ? (pf != y ? uint32_t(R) : uint32_t(U.part(uint32_t(pf)))) : 0u;
        const uint32_t rid = k2 < m ? uint32_t(U.part(k2)) : 0u;
        int32_t nl, nr;
        merge_rank2(T, pf >= 0, lid, uint32_t(R), k2 < m, uint32_t(R), rid, nl, nr);
        a.ws.lnl[s + j] = nl;
        a.ws.lnr[s + j] = nr;
        if (nl <= R || nr <= R) stop = min(stop, j);
      }
    }
    stop = uint32_t(block_min_i32(int32_t(min(stop, 0x7FFFFFFFu)), reinterpret_cast<int32_t *>(sh)));

    // 3. apply the merges up to and including `stop`
    for (uint32_t x = tid; x < 32 * nb && 2 * x <= stop; x += LONG_BLOCK) {
      const uint32_t b = x >> 5;
      const uint32_t two = uint32_t(U.sel[b] >> (2 * (x & 31))) & 3u;
      const uint32_t j = 64 * b + 2 * (x & 31) + ((two & 1) ? 0u : 1u);
      if (two && j <= stop) {
        const uint32_t k = U.next(j + 1);
        const uint32_t k2 = U.next(k + 1);
        const int y = U.prev(j);
        int pf = y;
        if (y >= 0) {
          const int z = U.prev(uint32_t(y));
          if (z >= 0 && U.chosen(uint32_t(z))) pf = z;
        }
        U.part(j) = R;
        U.rank(k) = RANK_NONE;
        if (pf >= 0) {
          U.rank(uint32_t(pf)) = a.ws.lnl[s + j];
          U.dirty[uint32_t(pf) >> 6] = 1;
        }
        // the pair to the right, unless the next part merges too (its own
        // left pair is then this part's right pair)
        if (!(k2 < m && k2 <= stop && U.chosen(k2))) U.rank(j) = a.ws.lnr[s + j];
        U.dirty[j >> 6] = 1;
        U.dirty[k >> 6] = 1;
      }
    }
    __syncthreads();
    // the merged right parts stop being part starts
    for (uint32_t x = tid; x < 32 * nb && 2 * x <= stop; x += LONG_BLOCK) {
      const uint32_t b = x >> 5;
      const uint32_t two = uint32_t(U.sel[b] >> (2 * (x & 31))) & 3u;
      const uint32_t j = 64 * b + 2 * (x & 31) + ((two & 1) ? 0u : 1u);
      if (two && j <= stop) {
        const uint32_t k = U.next(j + 1);
        atomicAnd(&U.bits[k >> 6], ~(1ull << (k & 63)));
      }
    }
    __syncthreads();
    for (uint32_t b = tid; b < nb; b += LONG_BLOCK) {
      U.sel[b] = 0;
      if (U.dirty[b]) {
        U.rescan(b);
        U.dirty[b] = 0;
      }
    }
    __syncthreads();
  }

  // output: ids in order; block counts scanned across threads
  uint32_t c = 0;
  for (uint32_t b0 = 0; b0 < nb; b0 += LONG_BLOCK) {
    const uint32_t b = b0 + tid;
    const unsigned long long A = b < nb ? U.bits[b] : 0ull;
    const uint32_t cnt = uint32_t(__popcll(A));
    uint32_t total;
    uint32_t o = c + block_excl_sum(cnt, sh, total);
    unsigned long long w = A;
    while (w) {
      const uint32_t t = uint32_t(__ffsll(w) - 1);
      w &= w - 1;
      a.ws.tmp_ids[s + o++] = U.part(64 * b + t);
    }
    c += total;
  }
  if (tid == 0) a.ws.piece_cnt[i] = c;
  __syncthreads();
}

// Merge of the units longer than WAVE_MAX, one workgroup each (its own
// kernel, on the second stream beside the short tier).
__global__ void __launch_bounds__(LONG_BLOCK) k_merge_long(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  __shared__ uint32_t sh[LONG_BLOCK];
  __shared__ LongLds ld;
  const uint32_t nll = a.ws.status->n_list[ML_LONG];
  for (uint32_t item = blockIdx.x; item < nll; item += gridDim.x)
    merge_long(a, a.ws.lst[ML_LONG][item], sh, ld);
}

// ---------------------------------------------------------------------------
// Ordered assembly: the exclusive scan of the units' id counts and the ids
// in output order, in one pass.  Each workgroup takes the next tile of
// ASM_UNITS units from a ticket counter (so a tile only ever waits for tiles
// whose workgroups are already running), publishes its own count, then
// reads its predecessors' published states from the nearest one back
// (decoupled look-back): a predecessor's prefix ends the walk, its count
// alone adds and moves on.  A state is one 64-bit word (flag and value
// together), written and read with agent-scope atomics, so no fence orders
// it.  Every wait is bounded: past SCAN_SPIN_MAX polls the call fails
// (status scan_fail) rather than wait on.
// ---------------------------------------------------------------------------
constexpr uint32_t ASM_BLOCK = 1024, ASM_PER = ASM_UNITS / ASM_BLOCK;  // 4 units per thread
constexpr unsigned long long SCAN_AGG = 1ull << 62, SCAN_PREFIX = 2ull << 62;
constexpr unsigned long long SCAN_VALUE = (1ull << 62) - 1;
constexpr uint32_t SCAN_SPIN_MAX = 1u << 22;

// ids of unit i: 1 for a unit settled by k_probe, else the count of the unit
// that merged its bytes (itself or its leader)
__device__ __forceinline__ uint32_t unit_count(const EncodeArgs &a, uint32_t i) {
  const int32_t u = a.ws.uid[i];
  if (u >= 0) return 1u;
  return a.ws.piece_cnt[u == UID_MERGED ? i : uint32_t(UID_FOLLOW - u)];
}

__device__ __forceinline__ void scan_publish(unsigned long long *p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long scan_read(unsigned long long *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The status block to pinned host memory (the call's result), all but
// scan_fail, which a failing tile sets there itself (the host clears it
// before each call).
__device__ __forceinline__ void publish_status(const EncodeArgs &a, Status *host) {
  publish_record(a, host, true);
}

// Texts above ASM_SINGLE_MAX bytes have more scan tiles than stay resident at
// once, and the look-back's waits grow with them; their tiles' sums are
// scanned apart instead: k_scan_sums (the sum of every tile), k_scan_bases
// (one workgroup: the exclusive scan of the sums), then k_assemble reads its
// base.
__global__ void __launch_bounds__(ASM_BLOCK) k_scan_sums(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  const uint32_t P = uint32_t(a.ws.status->n_pieces);
  const uint32_t t = blockIdx.x;
  if (t > P / ASM_UNITS) return;
  const uint32_t i0 = t * ASM_UNITS, nu = min(ASM_UNITS, P - i0);
  uint32_t sum = 0;
#pragma unroll
  for (uint32_t k = 0; k < ASM_PER; ++k) {
    const uint32_t j = k * ASM_BLOCK + threadIdx.x;
    if (j < nu) sum += unit_count(a, i0 + j);
  }
  __shared__ uint32_t s_w[ASM_BLOCK / 64];
  const uint32_t w = wave_sum(sum);
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x / 64] = w;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t tot = 0;
    for (uint32_t q = 0; q < ASM_BLOCK / 64; ++q) tot += s_w[q];
    a.ws.scan_state[t] = tot;
  }
}

__global__ void __launch_bounds__(1024) k_scan_bases(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  const uint32_t P = uint32_t(a.ws.status->n_pieces);
  const uint32_t T = P / ASM_UNITS + 1;
  const uint32_t tid = threadIdx.x, per = (T + 1023) / 1024;
  const uint32_t t0 = min(T, tid * per), t1 = min(T, t0 + per);
  unsigned long long sum = 0;
  for (uint32_t t = t0; t < t1; ++t) sum += a.ws.scan_state[t];
  __shared__ unsigned long long s_sum[33];
  unsigned long long total;
  unsigned long long run =
      block_incl_scan<1024>(sum, 0ull, [](unsigned long long x, unsigned long long y) { return x + y; },
                            s_sum, total) - sum;
  for (uint32_t t = t0; t < t1; ++t) {
    const unsigned long long v = a.ws.scan_state[t];
    a.ws.scan_state[t] = run;  // now the ids before tile t
    run += v;
  }
}

// single_pass: the tiles' bases by the look-back; else read from scan_state
// (k_scan_sums and k_scan_bases ran before).
struct AsmLds {
  uint32_t tile, excl, fail;
  uint32_t off[ASM_UNITS + 1], start[ASM_UNITS];
  int32_t uid[ASM_UNITS];
  uint32_t wsum[ASM_BLOCK / 64];
};

// One tile of the assembly; false when the look-back gave up (the call then
// reports a failure).
__device__ __forceinline__ bool assemble_tile(const EncodeArgs &a, Status *host, int single_pass,
                                              uint32_t t, uint32_t P, uint32_t nt, AsmLds &L) {
  Status *st = a.ws.status;
  uint32_t &s_excl = L.excl, &s_fail = L.fail;
  uint32_t *s_off = L.off, *s_start = L.start, *s_wsum = L.wsum;
  int32_t *s_uid = L.uid;
  const uint32_t i0 = t * ASM_UNITS;
  const uint32_t nu = min(ASM_UNITS, P - i0);  // units of this tile (the last may have 0)
  // counts: thread x takes units i0 + 4 x .. i0 + 4 x + 3; a unit's uid, its
  // count and its start load side by side (a follower of the word cache
  // needs its leader's count and start after)
  const uint32_t tid = threadIdx.x;
  int32_t uv[ASM_PER];
  uint32_t cnt[ASM_PER], sst[ASM_PER];
#pragma unroll
  for (uint32_t k = 0; k < ASM_PER; ++k) {
    const uint32_t j = tid * ASM_PER + k;
    const bool in = j < nu;
    uv[k] = in ? a.ws.uid[i0 + j] : 0;
    cnt[k] = in ? a.ws.piece_cnt[i0 + j] : 0u;
    sst[k] = in ? a.ws.piece_start[i0 + j] : 0u;
  }
#pragma unroll
  for (uint32_t k = 0; k < ASM_PER; ++k) {
    const int32_t u = uv[k];
    if (tid * ASM_PER + k >= nu) cnt[k] = 0u;
    else if (u >= 0) cnt[k] = 1u;
    else if (u != UID_MERGED) {
      const uint32_t src = uint32_t(UID_FOLLOW - u);
      cnt[k] = a.ws.piece_cnt[src];
      sst[k] = a.ws.piece_start[src];
    }
  }
  uint32_t sum = 0;
#pragma unroll
  for (uint32_t k = 0; k < ASM_PER; ++k) sum += cnt[k];
  // block scan of the per-thread sums
  const int lane = int(tid & 63);
  const uint32_t incl = wave_incl_sum(sum, lane);
  if (lane == 63) s_wsum[tid / 64] = incl;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (uint32_t q = 0; q < ASM_BLOCK / 64; ++q) {
    before += q < tid / 64 ? s_wsum[q] : 0u;
    total += s_wsum[q];
  }
  // the tile's place in the output: look-back by the first wave, 64
  // predecessors per step (lane l reads tile base - l); the nearest prefix
  // in the window ends the walk, else the window's counts add and it moves
  // 64 tiles back.  Before tile 0 reads as a prefix of 0.
  if (!single_pass) {
    if (tid == 0) {
      s_excl = uint32_t(a.ws.scan_state[t]);
      s_fail = 0;
    }
  } else if (tid < 64) {
    unsigned long long *state = a.ws.scan_state;
    if (tid == 0) scan_publish(&state[t], (t == 0 ? SCAN_PREFIX : SCAN_AGG) | total);
    unsigned long long acc = 0;
    uint32_t fail = 0;
    int64_t base = int64_t(t) - 1;
    for (;;) {  // wave-uniform
      const int64_t p = base - lane;
      unsigned long long v = p >= 0 ? scan_read(&state[p]) : SCAN_PREFIX;
      for (uint32_t spins = 0; __ballot(v == 0); ++spins) {
        if (spins >= SCAN_SPIN_MAX) {
          fail = 1;
          break;
        }
        if (v == 0) v = scan_read(&state[p]);
      }
      if (fail) break;
      const unsigned long long pm = __ballot((v & SCAN_PREFIX) != 0);
      const int f = pm ? __ffsll(pm) - 1 : 63;  // the nearest prefix, or the whole window
      unsigned long long x = lane <= f ? (v & SCAN_VALUE) : 0ull;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
      acc += x;
      if (pm) break;
      base -= 64;
    }
    if (tid == 0) {
      if (!fail && t > 0) scan_publish(&state[t], SCAN_PREFIX | (acc + total));
      s_excl = uint32_t(acc);
      s_fail = fail;
    }
  }
  __syncthreads();
  if (s_fail) {
    if (tid == 0) {
      host->scan_fail = 1u;
      __threadfence_system();
    }
    return false;
  }
  const uint32_t excl = s_excl;
  // unit offsets and sources into LDS
  uint32_t run = excl + before + incl - sum;
#pragma unroll
  for (uint32_t k = 0; k < ASM_PER; ++k) {
    const uint32_t j = tid * ASM_PER + k;
    if (j < nu) {
      s_off[j] = run;
      s_uid[j] = uv[k];
      s_start[j] = sst[k];
    }
    run += cnt[k];
  }
  if (tid == 0) s_off[nu] = excl + total;
  __syncthreads();
  // ids in output order: thread x writes ids o0 + x, o0 + x + 256, ..., each
  // finding its unit by a binary search over the tile's offsets (skipped
  // while the next id is in the same unit); nothing at or past the capacity
  const uint32_t o0 = excl, o1 = excl + total;
  const uint32_t cap = uint32_t(min<uint64_t>(a.ids_cap, 0xFFFFFFFFull));
  const uint32_t o1c = min(o1, cap);
  // (eight ids per round trip: their units found in LDS, then their loads
  // issued together, then their stores)
  constexpr uint32_t B = 8;
  uint32_t lo = 0, lo_end = 0;
  for (uint32_t ob = o0 + tid; ob < o1c; ob += B * ASM_BLOCK) {
    int32_t val[B];
    uint32_t src[B];
#pragma unroll
    for (uint32_t k = 0; k < B; ++k) {
      const uint32_t o = ob + k * ASM_BLOCK;
      src[k] = ~0u;
      val[k] = 0;
      if (o < o1c) {
        if (o >= lo_end) {
          uint32_t hi = nu;
          while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) >> 1;
            if (s_off[mid] <= o) lo = mid;
            else hi = mid;
          }
          lo_end = s_off[lo + 1];
        }
        const int32_t u = s_uid[lo];
        if (u >= 0) val[k] = u;
        else src[k] = s_start[lo] + (o - s_off[lo]);
      }
    }
#pragma unroll
    for (uint32_t k = 0; k < B; ++k)
      if (src[k] != ~0u) val[k] = a.ws.tmp_ids[src[k]];
#pragma unroll
    for (uint32_t k = 0; k < B; ++k) {
      const uint32_t o = ob + k * ASM_BLOCK;
      if (o < o1c) a.ids[o] = val[k];
    }
  }
  // id offset of every segment whose first unit (the first starting at or
  // after the segment's offset; index P for segments at the text's end) is
  // in this tile: segments with offsets in (start of unit i0 - 1, start of
  // the tile's last unit index]
  {
    const uint32_t iend = t + 1 == nt ? P : i0 + ASM_UNITS - 1;  // last unit index of the tile
    const uint64_t above = i0 == 0 ? 0ull : uint64_t(a.ws.piece_start[i0 - 1]) + 1;
    const uint64_t upto = iend >= P ? ~0ull : uint64_t(a.ws.piece_start[iend]);
    // first segment with offset >= above
    uint32_t s_lo = 0, hi = a.n_seg + 1;
    while (s_lo < hi) {
      const uint32_t mid = (s_lo + hi) >> 1;
      if (a.seg_off[mid] < above) s_lo = mid + 1;
      else hi = mid;
    }
    for (uint32_t s = s_lo + tid; s <= a.n_seg; s += ASM_BLOCK) {
      const uint64_t o = a.seg_off[s];
      if (o > upto) break;
      // first unit of the tile starting at or after o
      uint32_t l = 0, h = nu;
      while (l < h) {
        const uint32_t mid = (l + h) >> 1;
        if (a.ws.piece_start[i0 + mid] < o) l = mid + 1;
        else h = mid;
      }
      a.id_off[s] = int64_t(s_off[l]);
    }
  }
  if (t + 1 == nt && tid == 0) {
    // the last tile: the id total, the segment of the first UTF-8 error, and
    // the status block to the host
    st->n_ids = o1;
    const unsigned long long e = st->err_pos;
    if (e != ~0ull) {
      uint32_t l = 0, h = a.n_seg;
      while (l < h) {
        const uint32_t mid = (l + h) >> 1;
        if (a.seg_off[mid] <= e) l = mid + 1;
        else h = mid;
      }
      st->err_seg = l > 0 ? l - 1 : 0;
    }
    publish_status(a, host);
  }
  return true;
}

// Ordered assembly, single pass: each workgroup takes tiles from the ticket
// counter until none is left (a grid of a few workgroups per CU, not one per
// possible tile: the unit count is only known on the device, and a grid
// sized for the worst case spent most of its workgroups on exiting).
__global__ void __launch_bounds__(ASM_BLOCK) k_assemble(EncodeArgs a, Status *host) {
  Status *st = a.ws.status;
  if (st->pad2) {
    if (blockIdx.x == 0 && threadIdx.x == 0) publish_status(a, host);
    return;
  }
  const uint32_t P = uint32_t(st->n_pieces);
  const uint32_t nt = P / ASM_UNITS + 1;  // tiles over unit indices 0..P (P: the end)
  __shared__ AsmLds L;
  for (;;) {
    if (threadIdx.x == 0) L.tile = atomicAdd(&st->scan_ticket, 1u);
    __syncthreads();
    const uint32_t t = L.tile;
    if (t >= nt) return;
    if (!assemble_tile(a, host, 1, t, P, nt, L)) return;
    __syncthreads();  // the tile's LDS is read before the next tile writes it
  }
}

// The same after k_scan_sums and k_scan_bases (texts above ASM_SINGLE_MAX
// bytes): one tile per workgroup, its base read from the scan.
__global__ void __launch_bounds__(ASM_BLOCK) k_assemble_based(EncodeArgs a, Status *host) {
  Status *st = a.ws.status;
  if (st->pad2) {
    if (blockIdx.x == 0 && threadIdx.x == 0) publish_status(a, host);
    return;
  }
  const uint32_t P = uint32_t(st->n_pieces);
  const uint32_t nt = P / ASM_UNITS + 1;
  __shared__ AsmLds L;
  const uint32_t t = blockIdx.x;
  if (t >= nt) return;
  (void)assemble_tile(a, host, 0, t, P, nt, L);
}


}  // namespace bbpe
