// Back half of the encode path on gfx950: the list of merge units, byte-pair
// merging of every unit, and the ordered assembly of ids.
//
// The merge (tiktoken deep-dive page, "Inside encode"): ranks of adjacent
// pairs; repeatedly merge the lowest (leftmost on ties); recompute only the
// two pairs that touch the merged part.  A merged part's id is the rank that
// merged it; a part never merged is a single byte with its atom's rank.
// Three tiers by unit length:
//   short (<= 32 bytes): one lane per unit, bytes / pair ranks / part ids
//     in registers with static indexing;
//   mid (<= 1024 bytes): one wave per unit, state in LDS, argmin by a wave
//     reduction;
//   long: one wave per unit, state in global memory.
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
  __shared__ uint32_t s_sum[1024];
  const uint32_t T = a.n_tiles;
  const uint32_t tid = threadIdx.x;
  const uint32_t per = (T + 1023) / 1024;
  const uint32_t t0 = tid * per, t1 = min(T, t0 + per);
  uint32_t sum = 0;
  for (uint32_t t = t0; t < t1; ++t) sum += a.ws.tile_np[t];
  s_sum[tid] = sum;
  __syncthreads();
  for (uint32_t d = 1; d < 1024; d <<= 1) {
    uint32_t v = tid >= d ? s_sum[tid - d] : 0;
    __syncthreads();
    s_sum[tid] += v;
    __syncthreads();
  }
  uint32_t run = s_sum[tid] - sum;
  for (uint32_t t = t0; t < t1; ++t) {
    const uint32_t c = a.ws.tile_np[t];
    a.ws.tile_np[t] = run;
    run += c;
  }
  if (tid == 1023) {
    a.ws.tile_np[T] = s_sum[1023];
    a.ws.status->n_pieces = s_sum[1023];
    a.ws.piece_start[s_sum[1023]] = uint32_t(a.n);
  }
}

// unit start offsets, in text order
__global__ void __launch_bounds__(64) k_pieces(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  const int lane = threadIdx.x;
  const uint32_t t = blockIdx.x;
  const int64_t w = int64_t(t) * TILE_WORDS + lane - 1;
  const bool owned = lane >= 1 && lane <= int(TILE_WORDS) && w < int64_t(a.n_words);
  uint64_t ps = owned ? a.ws.ps[w] : 0;
  const uint32_t c = uint32_t(__popcll(ps));
  const uint32_t incl = wave_incl_sum(c, lane);
  uint32_t idx = a.ws.tile_np[t] + incl - c;
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

// Probe the table for a key with hash h, first word k8 and length len; the
// remaining bytes (for len > 8) are checked by `rest_eq(blob_ptr)`.
template <typename RestEq>
__device__ __forceinline__ int32_t probe(const DevTables &T, uint64_t h, uint64_t k8, uint32_t len,
                                         uint32_t &meta, RestEq rest_eq) {
  uint32_t idx = uint32_t(h) & T.slot_mask;
  for (;;) {
    const Slot s = T.slots[idx];
    if (s.rank < 0) return RANK_NONE;
    if ((s.meta & 0xFFu) == len && s.k8 == k8 &&
        (len <= 8 || rest_eq(T.blob + (s.meta >> META_OFF_SHIFT)))) {
      meta = s.meta;
      return s.rank;
    }
    idx = (idx + 1) & T.slot_mask;
  }
}

// Key = text bytes p[0..len).
__device__ __forceinline__ int32_t lookup_text(const DevTables &T, const uint8_t *__restrict__ p,
                                               uint32_t len, uint32_t &meta) {
  if (len > T.max_key_len) return RANK_NONE;
  uint64_t h = hash_seed(len);
  uint64_t k8 = 0;
  for (uint32_t i = 0; i < len; i += 8) {
    const uint32_t k = min(8u, len - i);
    uint64_t wv = 0;
    for (uint32_t j = 0; j < k; ++j) wv |= uint64_t(p[i + j]) << (8 * j);
    if (i == 0) k8 = wv;
    h = hash_step(h, wv);
  }
  return probe(T, h, k8, len, meta, [&](const uint8_t *b) {
    for (uint32_t j = 8; j < len; ++j)
      if (b[j] != p[j]) return false;
    return true;
  });
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
// Short tier: units of at most SK bytes, one lane each, in registers.
// ---------------------------------------------------------------------------
constexpr int SK = 32;
constexpr int SNB = SK / 4 + 3;  // dwords of unit bytes, with room for 8-byte slices
constexpr uint32_t MID_MAX = 1024;

struct UnitBytes {
  uint32_t d[SNB];
  __device__ __forceinline__ uint32_t byte(int j) const { return (d[j >> 2] >> (8 * (j & 3))) & 0xFFu; }
  // bytes a .. a+7 (a dynamic, a + 8 <= 4 * SNB)
  __device__ __forceinline__ uint64_t slice8(uint32_t a) const {
    const uint32_t q = a >> 2, o = a & 3u;
    uint32_t x0 = 0, x1 = 0, x2 = 0;
#pragma unroll
    for (int qq = 0; qq + 2 < SNB; ++qq) {
      const bool hit = uint32_t(qq) == q;
      x0 = hit ? d[qq] : x0;
      x1 = hit ? d[qq + 1] : x1;
      x2 = hit ? d[qq + 2] : x2;
    }
    const uint32_t lo = __builtin_amdgcn_alignbyte(x1, x0, o);
    const uint32_t hi = __builtin_amdgcn_alignbyte(x2, x1, o);
    return (uint64_t(hi) << 32) | lo;
  }
};

__device__ __forceinline__ uint32_t text_dword(const uint8_t *__restrict__ text, uint64_t n,
                                               uint64_t addr) {
  if (addr + 4 <= n) return *reinterpret_cast<const uint32_t *>(text + addr);
  uint32_t v = 0;
  for (uint32_t j = 0; j < 4; ++j)
    if (addr + j < n) v |= uint32_t(text[addr + j]) << (8 * j);
  return v;
}

// bytes [s, s+m) of the text, zero beyond m (m <= SK)
__device__ __forceinline__ void load_unit(const uint8_t *__restrict__ text, uint64_t n, uint32_t s,
                                          uint32_t m, UnitBytes &u) {
  const uint64_t a0 = s & ~3u;
  const uint32_t off = s & 3u;
  uint32_t raw[SNB + 1];
#pragma unroll
  for (int q = 0; q <= SNB; ++q) raw[q] = (4u * q < off + m) ? text_dword(text, n, a0 + 4u * q) : 0u;
#pragma unroll
  for (int q = 0; q < SNB; ++q) {
    const uint32_t v = __builtin_amdgcn_alignbyte(raw[q + 1], raw[q], off);
    const int lim = int(m) - 4 * q;
    const uint32_t keep = lim >= 4 ? 0xFFFFFFFFu : (lim <= 0 ? 0u : ((1u << (8 * lim)) - 1));
    u.d[q] = v & keep;
  }
}

__device__ __forceinline__ void unit_hash(const UnitBytes &u, uint32_t a, uint32_t len, uint64_t &h,
                                          uint64_t &k8) {
  h = hash_seed(len);
  k8 = 0;
  for (uint32_t i = 0; i < len; i += 8) {
    const uint64_t w = low_bytes(u.slice8(a + i), len - i);
    if (i == 0) k8 = w;
    h = hash_step(h, w);
  }
}

__device__ __forceinline__ bool unit_rest_eq(const UnitBytes &u, uint32_t a, uint32_t len,
                                             const uint8_t *b) {
  for (uint32_t i = 8; i < len; i += 8) {
    const uint32_t k = min(8u, len - i);
    uint64_t bw = 0;
    for (uint32_t j = 0; j < k; ++j) bw |= uint64_t(b[i + j]) << (8 * j);
    if (bw != low_bytes(u.slice8(a + i), k)) return false;
  }
  return true;
}

// Ranks of two keys of the unit, [a1, a1+l1) and [a2, a2+l2) (len 0 = none),
// with the first probes of both issued together.
__device__ __forceinline__ void unit_lookup2(const DevTables &T, const UnitBytes &u, uint32_t a1,
                                             uint32_t l1, uint32_t a2, uint32_t l2, int32_t &r1,
                                             int32_t &r2) {
  const bool v1 = l1 > 0 && l1 <= T.max_key_len, v2 = l2 > 0 && l2 <= T.max_key_len;
  uint64_t h1 = 0, k1 = 0, h2 = 0, k2 = 0;
  if (v1) unit_hash(u, a1, l1, h1, k1);
  if (v2) unit_hash(u, a2, l2, h2, k2);
  const uint32_t i1 = uint32_t(h1) & T.slot_mask, i2 = uint32_t(h2) & T.slot_mask;
  Slot s1{0, 0, -1}, s2{0, 0, -1};
  if (v1) s1 = T.slots[i1];
  if (v2) s2 = T.slots[i2];
  uint32_t meta;
  r1 = RANK_NONE;
  r2 = RANK_NONE;
  if (v1 && s1.rank >= 0) {
    if ((s1.meta & 0xFFu) == l1 && s1.k8 == k1 &&
        (l1 <= 8 || unit_rest_eq(u, a1, l1, T.blob + (s1.meta >> META_OFF_SHIFT))))
      r1 = s1.rank;
    else
      r1 = probe(T, h1 + 1, k1, l1, meta,
                 [&](const uint8_t *b) { return unit_rest_eq(u, a1, l1, b); });
  }
  if (v2 && s2.rank >= 0) {
    if ((s2.meta & 0xFFu) == l2 && s2.k8 == k2 &&
        (l2 <= 8 || unit_rest_eq(u, a2, l2, T.blob + (s2.meta >> META_OFF_SHIFT))))
      r2 = s2.rank;
    else
      r2 = probe(T, h2 + 1, k2, l2, meta,
                 [&](const uint8_t *b) { return unit_rest_eq(u, a2, l2, b); });
  }
}

__device__ __forceinline__ uint32_t above32(int j) { return ~((2u << j) - 1u); }

// Merge a unit of 2 <= m <= SK bytes; writes its ids to out, returns their count.
__device__ __forceinline__ uint32_t merge_short(const DevTables &T, const UnitBytes &u, uint32_t m,
                                                int32_t *out) {
  int32_t r[SK], pr[SK];
#pragma unroll
  for (int j = 0; j < SK; ++j) {
    const uint32_t b0 = u.byte(j), b1 = (j + 1 < SK) ? u.byte(j + 1) : 0u;
    r[j] = (uint32_t(j) + 1 < m) ? T.pair[b0 * 256u + b1] : RANK_NONE;
    pr[j] = (uint32_t(j) < m) ? T.atom[b0] : 0;
  }
  uint32_t bnd = (m >= 32) ? 0xFFFFFFFFu : ((1u << m) - 1u);
  for (uint32_t round = 0; round + 1 < m; ++round) {
    int32_t best = RANK_NONE;
    int bj = 0;
#pragma unroll
    for (int j = 0; j < SK; ++j) {
      const bool lt = r[j] < best;  // strict: the leftmost minimum wins
      best = lt ? r[j] : best;
      bj = lt ? j : bj;
    }
    if (best == RANK_NONE) break;
    const int k = __ffs(bnd & above32(bj)) - 1;  // the part merged into bj
    bnd &= ~(1u << k);
    const uint32_t after = bnd & above32(bj);
    const uint32_t k2 = after ? uint32_t(__ffs(after) - 1) : m;  // end of the merged part
    const uint32_t rest = after & (after - 1);
    const uint32_t end2 = rest ? uint32_t(__ffs(rest) - 1) : m;
    const uint32_t before = bnd & ((1u << bj) - 1u);
    const int q = before ? 31 - __clz(before) : -1;
    int32_t nb, nq;
    unit_lookup2(T, u, uint32_t(bj), after ? end2 - uint32_t(bj) : 0u, uint32_t(q < 0 ? 0 : q),
                 q >= 0 ? k2 - uint32_t(q) : 0u, nb, nq);
#pragma unroll
    for (int j = 0; j < SK; ++j) {
      r[j] = (j == k) ? RANK_NONE : r[j];
      r[j] = (j == bj) ? nb : r[j];
      pr[j] = (j == bj) ? best : pr[j];
      r[j] = (j == q) ? nq : r[j];
    }
  }
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < SK; ++j)
    if ((bnd >> j) & 1u) out[c++] = pr[j];
  return c;
}

__global__ void __launch_bounds__(64) k_merge(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  const uint32_t P = uint32_t(a.ws.status->n_pieces);
  const DevTables &T = a.T;
  for (uint32_t i = blockIdx.x * 64 + threadIdx.x; i < P; i += gridDim.x * 64) {
    const uint32_t s = a.ws.piece_start[i];
    const uint32_t m = a.ws.piece_start[i + 1] - s;
    int32_t *out = a.ws.tmp_ids + s;
    if ((a.ws.spst[s >> 6] >> (s & 63)) & 1) {
      out[0] = special_id(T, a.text + s, m);
      a.ws.piece_cnt[i] = 1;
      continue;
    }
    if (m == 1) {
      out[0] = T.atom[a.text[s]];
      a.ws.piece_cnt[i] = 1;
      continue;
    }
    if (m > uint32_t(SK)) {
      uint32_t meta = 0;
      const int32_t r = lookup_text(T, a.text + s, m, meta);
      if (r != RANK_NONE && (meta & META_SELF)) {
        out[0] = r;
        a.ws.piece_cnt[i] = 1;
      } else if (m <= MID_MAX) {
        a.ws.mid_list[atomicAdd(&a.ws.status->n_mid, 1u)] = i;
      } else {
        a.ws.long_list[atomicAdd(&a.ws.status->n_long, 1u)] = i;
      }
      continue;
    }
    UnitBytes u;
    load_unit(a.text, a.n, s, m, u);
    // a unit that is itself a key whose own merges rebuild it
    uint64_t h, k8;
    unit_hash(u, 0, m, h, k8);
    uint32_t meta = 0;
    const int32_t r = probe(T, h, k8, m, meta,
                            [&](const uint8_t *b) { return unit_rest_eq(u, 0, m, b); });
    if (r != RANK_NONE && (meta & META_SELF)) {
      out[0] = r;
      a.ws.piece_cnt[i] = 1;
      continue;
    }
    a.ws.piece_cnt[i] = merge_short(T, u, m, out);
  }
}

// ---------------------------------------------------------------------------
// Wave tiers
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    unsigned long long o = __shfl_xor(v, d, 64);
    v = o < v ? o : v;
  }
  return v;
}

// Mid tier: one wave per unit of at most MID_MAX bytes, all state in LDS.
__global__ void __launch_bounds__(64) k_merge_mid(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  __shared__ uint8_t s_b[MID_MAX];
  __shared__ int32_t s_r[MID_MAX];
  __shared__ int32_t s_pr[MID_MAX];
  __shared__ unsigned long long s_alive[MID_MAX / 64];
  const int lane = threadIdx.x;
  const uint32_t nm = a.ws.status->n_mid;
  const DevTables &T = a.T;
  for (uint32_t li = blockIdx.x; li < nm; li += gridDim.x) {
    const uint32_t i = a.ws.mid_list[li];
    const uint32_t s = a.ws.piece_start[i];
    const uint32_t m = a.ws.piece_start[i + 1] - s;
    const uint32_t nw = (m + 63) / 64;
    for (uint32_t j = uint32_t(lane); j < m; j += 64) s_b[j] = a.text[s + j];
    __syncthreads();
    for (uint32_t j = uint32_t(lane); j < m; j += 64) {
      s_r[j] = (j + 1 < m) ? T.pair[uint32_t(s_b[j]) * 256u + s_b[j + 1]] : RANK_NONE;
      s_pr[j] = T.atom[s_b[j]];
    }
    for (uint32_t wd = uint32_t(lane); wd < nw; wd += 64) {
      const uint32_t left = m - wd * 64;
      s_alive[wd] = left >= 64 ? ~0ull : ((1ull << left) - 1);
    }
    __syncthreads();
    // next / previous part start after / before position p (parts are keys,
    // at most BBPE_MAX_KEY_BYTES long, so at most three words are read)
    auto next_alive = [&](uint32_t p) -> uint32_t {
      uint32_t x = p + 1;
      while (x < m) {
        const uint32_t wd = x >> 6;
        const unsigned long long bits = s_alive[wd] & (~0ull << (x & 63));
        if (bits) return wd * 64 + uint32_t(__ffsll(bits) - 1);
        x = (wd + 1) * 64;
      }
      return m;
    };
    auto prev_alive = [&](uint32_t p) -> int {
      int x = int(p) - 1;
      while (x >= 0) {
        const uint32_t wd = uint32_t(x) >> 6;
        const unsigned long long msk = (x & 63) == 63 ? ~0ull : ((1ull << ((x & 63) + 1)) - 1);
        const unsigned long long bits = s_alive[wd] & msk;
        if (bits) return int(wd * 64 + 63 - __clzll(bits));
        x = int(wd * 64) - 1;
      }
      return -1;
    };
    for (uint32_t round = 0; round + 1 < m; ++round) {
      unsigned long long key = ~0ull;
      for (uint32_t j = uint32_t(lane); j < m; j += 64) {
        const int32_t rv = s_r[j];
        const unsigned long long kk =
            rv == RANK_NONE ? ~0ull : ((static_cast<unsigned long long>(uint32_t(rv)) << 32) | j);
        key = kk < key ? kk : key;
      }
      key = wave_min_u64(key);
      if (key == ~0ull) break;
      const int32_t best = int32_t(key >> 32);
      const uint32_t bj = uint32_t(key & 0xffffffffu);
      const uint32_t k = next_alive(bj);
      const uint32_t k2 = next_alive(k);  // start of the part after the merged one
      const uint32_t end2 = (k2 < m) ? next_alive(k2) : m;
      const int q = prev_alive(bj);
      // lane 0 looks up the merged part with its right neighbour, lane 1 the
      // left neighbour with the merged part
      int32_t rv = RANK_NONE;
      uint32_t meta;
      if (lane == 0 && k2 < m) rv = lookup_text(T, a.text + s + bj, end2 - bj, meta);
      if (lane == 1 && q >= 0) rv = lookup_text(T, a.text + s + uint32_t(q), k2 - uint32_t(q), meta);
      const int32_t nb = __shfl(rv, 0, 64), nq = __shfl(rv, 1, 64);
      __syncthreads();
      if (lane == 0) {
        s_alive[k >> 6] &= ~(1ull << (k & 63));
        s_r[k] = RANK_NONE;
        s_r[bj] = nb;
        s_pr[bj] = best;
        if (q >= 0) s_r[q] = nq;
      }
      __syncthreads();
    }
    uint32_t c = 0;
    for (uint32_t j0 = 0; j0 < m; j0 += 64) {
      const uint32_t j = j0 + uint32_t(lane);
      const bool hit = j < m && ((s_alive[j >> 6] >> (j & 63)) & 1);
      const unsigned long long bal = __ballot(hit);
      if (hit) a.ws.tmp_ids[s + c + uint32_t(__popcll(bal & ((1ull << lane) - 1)))] = s_pr[j];
      c += uint32_t(__popcll(bal));
    }
    if (lane == 0) a.ws.piece_cnt[i] = c;
    __syncthreads();
  }
}

// Long tier: one wave per unit longer than MID_MAX.  Arrays indexed by text
// byte position (units never overlap): lrank = pair rank at a part start,
// lpart = id of the part starting there, lalive = 1 where a part starts;
// per-64-byte-block minima of (rank << 32 | offset) in lmin, at index
// s/32 + block (a unit of m > 64 bytes needs ceil(m/64) <= floor(m/32)
// entries, so units never share one).  Lane 0 applies each merge;
// device-scope fences make its stores visible to the other lanes.
__device__ __forceinline__ bool alive(const EncodeArgs &a, uint32_t pos) {
  return a.ws.lalive[pos] != 0;
}

// minimum key over the parts of local block blk of the unit [s, s+m)
__device__ __forceinline__ unsigned long long block_min(const EncodeArgs &a, uint32_t s, uint32_t m,
                                                        uint32_t blk, int lane) {
  const uint32_t j = blk * 64 + uint32_t(lane);
  unsigned long long key = ~0ull;
  if (j < m && alive(a, s + j)) {
    const int32_t r = a.ws.lrank[s + j];
    if (r != RANK_NONE) key = (static_cast<unsigned long long>(uint32_t(r)) << 32) | j;
  }
  return wave_min_u64(key);
}

__global__ void __launch_bounds__(64) k_merge_long(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  const int lane = threadIdx.x;
  const uint32_t nl = a.ws.status->n_long;
  const DevTables &T = a.T;
  for (uint32_t li = blockIdx.x; li < nl; li += gridDim.x) {
    const uint32_t i = a.ws.long_list[li];
    const uint32_t s = a.ws.piece_start[i];
    const uint32_t m = a.ws.piece_start[i + 1] - s;
    const uint8_t *p = a.text + s;
    unsigned long long *lmin = a.ws.lmin + (s >> 5);
    const uint32_t nblk = (m + 63) / 64;
    for (uint32_t j = uint32_t(lane); j < m; j += 64) {
      a.ws.lrank[s + j] = (j + 1 < m) ? T.pair[uint32_t(p[j]) * 256u + p[j + 1]] : RANK_NONE;
      a.ws.lpart[s + j] = T.atom[p[j]];
      a.ws.lalive[s + j] = 1;
    }
    __threadfence();
    for (uint32_t b = 0; b < nblk; ++b) {
      const unsigned long long v = block_min(a, s, m, b, lane);
      if (lane == 0) lmin[b] = v;
    }
    __threadfence();
    // every round removes one part, so at most m - 1 rounds
    for (uint32_t round = 0; round + 1 < m; ++round) {
      unsigned long long key = ~0ull;
      for (uint32_t b = uint32_t(lane); b < nblk; b += 64) {
        const unsigned long long v = lmin[b];
        key = v < key ? v : key;
      }
      key = wave_min_u64(key);
      if (key == ~0ull) break;
      const int32_t best = int32_t(key >> 32);
      const uint32_t bj = uint32_t(key & 0xffffffffu);
      // the part after bj starts within BBPE_MAX_KEY_BYTES (parts are keys)
      uint32_t k = m;
      for (uint32_t off = 1; off <= BBPE_MAX_KEY_BYTES + 1 && k == m; off += 64) {
        const uint32_t j = bj + off + uint32_t(lane);
        const unsigned long long bal = __ballot(j < m && alive(a, s + j));
        if (bal) k = bj + off + uint32_t(__ffsll(bal) - 1);
      }
      if (k >= m) break;  // cannot happen: a ranked pair has a right part
      uint32_t k2 = m;
      for (uint32_t off = 1; off <= BBPE_MAX_KEY_BYTES + 1 && k2 == m; off += 64) {
        const uint32_t j = k + off + uint32_t(lane);
        const unsigned long long bal = __ballot(j < m && alive(a, s + j));
        if (bal) k2 = k + off + uint32_t(__ffsll(bal) - 1);
      }
      uint32_t end2 = m;
      if (k2 < m) {
        for (uint32_t off = 1; off <= BBPE_MAX_KEY_BYTES + 1 && end2 == m; off += 64) {
          const uint32_t j = k2 + off + uint32_t(lane);
          const unsigned long long bal = __ballot(j < m && alive(a, s + j));
          if (bal) end2 = k2 + off + uint32_t(__ffsll(bal) - 1);
        }
      }
      uint32_t q = m;
      for (uint32_t off = 1; off <= BBPE_MAX_KEY_BYTES + 1 && q == m; off += 64) {
        const int64_t j = int64_t(bj) - int64_t(off) - lane;
        const unsigned long long bal = __ballot(j >= 0 && alive(a, s + uint32_t(j)));
        if (bal) q = bj - off - uint32_t(__ffsll(bal) - 1);
      }
      int32_t rv = RANK_NONE;
      uint32_t meta;
      if (lane == 0 && k2 < m) rv = lookup_text(T, p + bj, end2 - bj, meta);
      if (lane == 1 && q < m) rv = lookup_text(T, p + q, k2 - q, meta);
      const int32_t nb = __shfl(rv, 0, 64), nq = __shfl(rv, 1, 64);
      if (lane == 0) {
        a.ws.lalive[s + k] = 0;
        a.ws.lpart[s + bj] = best;
        a.ws.lrank[s + bj] = nb;
        if (q < m) a.ws.lrank[s + q] = nq;
        a.ws.lrank[s + k] = RANK_NONE;
      }
      __threadfence();
      const uint32_t b0 = bj / 64, bk = k / 64, bq = (q < m) ? q / 64 : b0;
      unsigned long long v = block_min(a, s, m, b0, lane);
      if (lane == 0) lmin[b0] = v;
      if (bk != b0) {
        v = block_min(a, s, m, bk, lane);
        if (lane == 0) lmin[bk] = v;
      }
      if (bq != b0 && bq != bk) {
        v = block_min(a, s, m, bq, lane);
        if (lane == 0) lmin[bq] = v;
      }
      __threadfence();
    }
    uint32_t c = 0;
    for (uint32_t j0 = 0; j0 < m; j0 += 64) {
      const uint32_t j = j0 + uint32_t(lane);
      const bool hit = j < m && alive(a, s + j);
      const unsigned long long bal = __ballot(hit);
      if (hit) a.ws.tmp_ids[s + c + uint32_t(__popcll(bal & ((1ull << lane) - 1)))] = a.ws.lpart[s + j];
      c += uint32_t(__popcll(bal));
    }
    if (lane == 0) a.ws.piece_cnt[i] = c;
  }
}

// ---------------------------------------------------------------------------
// Exclusive scan of ids per unit (three phases, 4096 units per block).
// ---------------------------------------------------------------------------
constexpr uint32_t SCAN_BLOCK = 256, SCAN_ITEMS = 16, SCAN_TILE = SCAN_BLOCK * SCAN_ITEMS;

__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *sh, uint32_t &total) {
  const uint32_t tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (uint32_t d = 1; d < SCAN_BLOCK; d <<= 1) {
    const uint32_t o = tid >= d ? sh[tid - d] : 0;
    __syncthreads();
    sh[tid] += o;
    __syncthreads();
  }
  total = sh[SCAN_BLOCK - 1];
  const uint32_t r = sh[tid] - v;
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(SCAN_BLOCK) k_scan_reduce(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  __shared__ uint32_t sh[SCAN_BLOCK];
  const uint32_t P = uint32_t(a.ws.status->n_pieces);
  const uint32_t b0 = blockIdx.x * SCAN_TILE;
  if (b0 >= P + 1) return;
  uint32_t sum = 0;
  for (uint32_t k = 0; k < SCAN_ITEMS; ++k) {
    const uint32_t i = b0 + threadIdx.x * SCAN_ITEMS + k;
    if (i < P) sum += a.ws.piece_cnt[i];
  }
  uint32_t total;
  block_excl_scan(sum, sh, total);
  if (threadIdx.x == 0) a.ws.scan_part[blockIdx.x] = total;
}

__global__ void __launch_bounds__(1024) k_scan_partials(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  __shared__ uint32_t sh[1024];
  const uint32_t P = uint32_t(a.ws.status->n_pieces);
  const uint32_t nb = (P + 1 + SCAN_TILE - 1) / SCAN_TILE;
  const uint32_t tid = threadIdx.x;
  const uint32_t per = (nb + 1023) / 1024;
  const uint32_t t0 = tid * per, t1 = min(nb, t0 + per);
  uint32_t sum = 0;
  for (uint32_t t = t0; t < t1; ++t) sum += a.ws.scan_part[t];
  sh[tid] = sum;
  __syncthreads();
  for (uint32_t d = 1; d < 1024; d <<= 1) {
    const uint32_t o = tid >= d ? sh[tid - d] : 0;
    __syncthreads();
    sh[tid] += o;
    __syncthreads();
  }
  uint32_t run = sh[tid] - sum;
  for (uint32_t t = t0; t < t1; ++t) {
    const uint32_t c = a.ws.scan_part[t];
    a.ws.scan_part[t] = run;
    run += c;
  }
}

__global__ void __launch_bounds__(SCAN_BLOCK) k_scan_down(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  __shared__ uint32_t sh[SCAN_BLOCK];
  const uint32_t P = uint32_t(a.ws.status->n_pieces);
  const uint32_t b0 = blockIdx.x * SCAN_TILE;
  if (b0 >= P + 1) return;
  uint32_t v[SCAN_ITEMS];
  uint32_t sum = 0;
  for (uint32_t k = 0; k < SCAN_ITEMS; ++k) {
    const uint32_t i = b0 + threadIdx.x * SCAN_ITEMS + k;
    v[k] = i < P ? a.ws.piece_cnt[i] : 0u;
    sum += v[k];
  }
  uint32_t total;
  uint32_t run = block_excl_scan(sum, sh, total) + a.ws.scan_part[blockIdx.x];
  for (uint32_t k = 0; k < SCAN_ITEMS; ++k) {
    const uint32_t i = b0 + threadIdx.x * SCAN_ITEMS + k;
    if (i <= P) a.ws.piece_cnt[i] = run;  // piece_cnt[P] becomes the total
    run += v[k];
  }
}

// ids in order: unit i's ids go to [id_base[i], id_base[i+1])
__global__ void __launch_bounds__(256) k_assemble(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  const uint32_t P = uint32_t(a.ws.status->n_pieces);
  const uint32_t total = P ? a.ws.piece_cnt[P] : 0u;
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < P; i += gridDim.x * 256) {
    const uint32_t o = a.ws.piece_cnt[i], e = a.ws.piece_cnt[i + 1];
    const uint32_t s = a.ws.piece_start[i];
    if (e <= a.ids_cap)
      for (uint32_t j = 0; j < e - o; ++j) a.ids[o + j] = a.ws.tmp_ids[s + j];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) a.ws.status->n_ids = total;
}

// id offset of every segment, and the segment of the first UTF-8 error
__global__ void __launch_bounds__(256) k_seg_offsets(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  const uint32_t P = uint32_t(a.ws.status->n_pieces);
  for (uint32_t s = blockIdx.x * 256 + threadIdx.x; s <= a.n_seg; s += gridDim.x * 256) {
    const uint64_t o = a.seg_off[s];
    // first unit starting at or after o
    uint32_t lo = 0, hi = P;
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if (a.ws.piece_start[mid] < o) lo = mid + 1;
      else hi = mid;
    }
    a.id_off[s] = P ? int64_t(a.ws.piece_cnt[lo]) : 0;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const unsigned long long e = a.ws.status->err_pos;
    if (e != ~0ull) {
      uint32_t lo = 0, hi = a.n_seg;
      while (lo < hi) {
        const uint32_t mid = (lo + hi) >> 1;
        if (a.seg_off[mid] <= e) lo = mid + 1;
        else hi = mid;
      }
      a.ws.status->err_seg = lo > 0 ? lo - 1 : 0;
    }
  }
}

}  // namespace bbpe
