// Back half of the encode path on gfx950: the list of pieces, byte-pair
// merging of every piece, and the ordered assembly of ids.
#include <hip/hip_runtime.h>

#include "bbpe_device.h"
#include "bbpe_kernels.h"

namespace bbpe {

// ---------------------------------------------------------------------------
// Piece list
// ---------------------------------------------------------------------------
// one workgroup: exclusive scan of pieces per tile; the total becomes P
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

// piece start offsets, in text order
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
// Rank of the byte string p[0..len) (a slice of the text), or RANK_NONE.
// meta receives the slot's metadata on a hit.
__device__ __forceinline__ int32_t lookup(const DevTables &T, const uint8_t *__restrict__ p,
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
  uint32_t idx = uint32_t(h) & T.slot_mask;
  for (;;) {
    const Slot s = T.slots[idx];
    if (s.rank < 0) return RANK_NONE;
    if ((s.meta & 0xFFu) == len && s.k8 == k8) {
      bool eq = true;
      if (len > 8) {
        const uint8_t *b = T.blob + (s.meta >> META_OFF_SHIFT);
        for (uint32_t j = 8; j < len && eq; ++j) eq = b[j] == p[j];
      }
      if (eq) {
        meta = s.meta;
        return s.rank;
      }
    }
    idx = (idx + 1) & T.slot_mask;
  }
}

__device__ __forceinline__ int32_t rank_of(const DevTables &T, const uint8_t *p, uint32_t len) {
  uint32_t meta;
  return lookup(T, p, len, meta);
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
// Merge (tiktoken deep-dive page, "Inside encode"): ranks of adjacent pairs,
// repeatedly merge the lowest (leftmost on ties), recompute only the pairs
// that touch the merged part.  A merged part's id is the rank that merged it.
// Pieces of at most 64 bytes: one lane each, parts as a 64-bit mask of their
// start bytes, pair ranks and part ids in LDS.  Longer pieces go to a list
// for the wave-per-piece tier.
// ---------------------------------------------------------------------------
constexpr int MERGE_BLOCK = 64;
constexpr uint32_t SHORT_MAX = 64;

__device__ __forceinline__ uint64_t above(int j) { return ~((uint64_t(2) << j) - 1); }

__global__ void __launch_bounds__(MERGE_BLOCK) k_merge(EncodeArgs a) {
  if (a.ws.status->pad2) return;
  __shared__ int32_t s_r[SHORT_MAX * MERGE_BLOCK];
  __shared__ int32_t s_pr[SHORT_MAX * MERGE_BLOCK];
  const uint32_t tid = threadIdx.x;
  const uint32_t P = uint32_t(a.ws.status->n_pieces);
  const DevTables &T = a.T;
  for (uint32_t i = blockIdx.x * MERGE_BLOCK + tid; i < P; i += gridDim.x * MERGE_BLOCK) {
    const uint32_t s = a.ws.piece_start[i];
    const uint32_t m = a.ws.piece_start[i + 1] - s;
    const uint8_t *p = a.text + s;
    int32_t *out = a.ws.tmp_ids + s;
    if ((a.ws.spst[s >> 6] >> (s & 63)) & 1) {
      out[0] = special_id(T, p, m);
      a.ws.piece_cnt[i] = 1;
      continue;
    }
    if (m == 1) {
      out[0] = T.atom[p[0]];
      a.ws.piece_cnt[i] = 1;
      continue;
    }
    {
      // a piece that is itself a key whose own merges rebuild it
      uint32_t meta = 0;
      const int32_t r = lookup(T, p, m, meta);
      if (r != RANK_NONE && (meta & META_SELF)) {
        out[0] = r;
        a.ws.piece_cnt[i] = 1;
        continue;
      }
    }
    if (m > SHORT_MAX) {
      const uint32_t k = atomicAdd(&a.ws.status->n_long, 1u);
      a.ws.long_list[k] = i;
      continue;
    }
#define R_(j) s_r[(j) * MERGE_BLOCK + tid]
#define PR_(j) s_pr[(j) * MERGE_BLOCK + tid]
    for (uint32_t j = 0; j + 1 < m; ++j) {
      R_(j) = T.pair[uint32_t(p[j]) * 256u + p[j + 1]];
      PR_(j) = T.atom[p[j]];
    }
    R_(m - 1) = RANK_NONE;
    PR_(m - 1) = T.atom[p[m - 1]];
    uint64_t bnd = (m == 64) ? ~uint64_t(0) : (bit(int(m)) - 1);
    for (;;) {
      int32_t best = RANK_NONE;
      int bj = -1;
      for (uint64_t x = bnd; x; x &= x - 1) {
        const int j = __ffsll(static_cast<unsigned long long>(x)) - 1;
        const int32_t rv = R_(j);
        if (rv < best) {
          best = rv;
          bj = j;
        }
      }
      if (best == RANK_NONE) break;
      const int k = __ffsll(static_cast<unsigned long long>(bnd & above(bj))) - 1;
      bnd &= ~bit(k);
      PR_(bj) = best;
      const uint64_t after = bnd & above(bj);
      const uint32_t endbj = after ? uint32_t(__ffsll(static_cast<unsigned long long>(after)) - 1) : m;
      if (after) {
        const uint64_t rest = after & (after - 1);
        const uint32_t end2 = rest ? uint32_t(__ffsll(static_cast<unsigned long long>(rest)) - 1) : m;
        R_(bj) = rank_of(T, p + bj, end2 - uint32_t(bj));
      } else {
        R_(bj) = RANK_NONE;
      }
      const uint64_t before = bnd & (bit(bj) - 1);
      if (before) {
        const int q = 63 - __clzll(before);
        R_(q) = rank_of(T, p + q, endbj - uint32_t(q));
      }
    }
    uint32_t c = 0;
    for (uint64_t x = bnd; x; x &= x - 1) {
      const int j = __ffsll(static_cast<unsigned long long>(x)) - 1;
      out[c++] = PR_(j);
    }
    a.ws.piece_cnt[i] = c;
#undef R_
#undef PR_
  }
}

// Long pieces: one wave per piece.  Arrays indexed by text byte position
// (pieces never overlap): lrank = pair rank at a part start, lpart = id of
// the part starting there, lalive = 1 where a part starts; per-64-byte-block
// minima of (rank << 32 | offset) in lmin, at index s/32 + block (a piece of
// m > 64 bytes needs ceil(m/64) <= floor(m/32) entries, so pieces never
// share one).  Lane 0 applies each merge; device-scope fences make its
// stores visible to the other lanes before they read.
__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    unsigned long long o = __shfl_xor(v, d, 64);
    v = o < v ? o : v;
  }
  return v;
}

__device__ __forceinline__ bool alive(const EncodeArgs &a, uint32_t pos) {
  return a.ws.lalive[pos] != 0;
}

// minimum key over the parts of local block blk of the piece [s, s+m)
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
    }
    // all bytes start as parts
    for (uint32_t j = uint32_t(lane); j < m; j += 64) a.ws.lalive[s + j] = 1;
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
      // the part after bj starts within 128 bytes (parts are keys)
      uint32_t k = m;
      for (uint32_t off = 1; off <= BBPE_MAX_KEY_BYTES + 1 && k == m; off += 64) {
        const uint32_t j = bj + off + uint32_t(lane);
        const bool hit = j < m && alive(a, s + j);
        const unsigned long long bal = __ballot(hit);
        if (bal) k = bj + off + uint32_t(__ffsll(bal) - 1);
      }
      if (k >= m) break;  // cannot happen: a ranked pair has a right part
      // part after k (new right neighbour) and the one after it
      uint32_t k2 = m;
      for (uint32_t off = 1; off <= BBPE_MAX_KEY_BYTES + 1 && k2 == m; off += 64) {
        const uint32_t j = k + off + uint32_t(lane);
        const bool hit = j < m && alive(a, s + j);
        const unsigned long long bal = __ballot(hit);
        if (bal) k2 = k + off + uint32_t(__ffsll(bal) - 1);
      }
      uint32_t end2 = m;
      if (k2 < m) {
        for (uint32_t off = 1; off <= BBPE_MAX_KEY_BYTES + 1 && end2 == m; off += 64) {
          const uint32_t j = k2 + off + uint32_t(lane);
          const bool hit = j < m && alive(a, s + j);
          const unsigned long long bal = __ballot(hit);
          if (bal) end2 = k2 + off + uint32_t(__ffsll(bal) - 1);
        }
      }
      // part before bj
      uint32_t q = m;
      for (uint32_t off = 1; off <= BBPE_MAX_KEY_BYTES + 1 && q == m; off += 64) {
        const int64_t j = int64_t(bj) - int64_t(off) - lane;
        const bool hit = j >= 0 && alive(a, s + uint32_t(j));
        const unsigned long long bal = __ballot(hit);
        if (bal) q = bj - off - uint32_t(__ffsll(bal) - 1);
      }
      if (lane == 0) {
        a.ws.lalive[s + k] = 0;
        a.ws.lpart[s + bj] = best;
        a.ws.lrank[s + bj] = (k2 < m) ? rank_of(T, p + bj, end2 - bj) : RANK_NONE;
        if (q < m) a.ws.lrank[s + q] = rank_of(T, p + q, k2 - q);
        a.ws.lrank[s + k] = RANK_NONE;
      }
      __threadfence();
      // refresh the block minima that changed
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
    // write the surviving parts in order
    uint32_t c = 0;
    for (uint32_t j0 = 0; j0 < m; j0 += 64) {
      const uint32_t j = j0 + uint32_t(lane);
      const bool hit = j < m && alive(a, s + j);
      const unsigned long long bal = __ballot(hit);
      if (hit) {
        const uint32_t rank_in = uint32_t(__popcll(bal & ((1ull << lane) - 1)));
        a.ws.tmp_ids[s + c + rank_in] = a.ws.lpart[s + j];
      }
      c += uint32_t(__popcll(bal));
    }
    if (lane == 0) a.ws.piece_cnt[i] = c;
  }
}

// ---------------------------------------------------------------------------
// Exclusive scan of ids per piece (three phases, 4096 pieces per block).
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

// ids in order: piece i's ids go to [id_base[i], id_base[i+1])
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
    // first piece starting at or after o
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
