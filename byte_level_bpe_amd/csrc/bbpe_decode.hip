// Decode on the device (gfx950): ids to bytes, each token's bytes gathered
// at its offset in the output, the offsets being the exclusive scan of the
// tokens' byte lengths (tiktoken deep-dive page, "An encoding is three
// objects": decoding concatenates the tokens' bytes; specials decode to
// their strings).  The same offsets are each token's byte offset in the text
// it was encoded from, an optional output.  The tail check reports how much
// of the output ends on a complete UTF-8 character, so that a streaming
// caller can hold the rest back (a token may end inside a character).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "../../include/bbpe.h"
#include "bbpe_device.h"
#include "bbpe_internal.h"
#include "bbpe_launch.h"
#include "bbpe_tokenizer.h"

namespace bbpe {
namespace {

constexpr uint32_t DEC_BLOCK = 256, DEC_ITEMS = 16, DEC_TILE = DEC_BLOCK * DEC_ITEMS;

struct DecStatus {
  unsigned long long first_bad;  // index of the first id that is neither rank nor special, or ~0
  unsigned long long total;      // output bytes
  unsigned long long complete;   // bytes up to the end of the last complete character
  unsigned long long pad;
};

struct DecArgs {
  DevTables T;
  const int32_t *ids;
  uint64_t n;
  uint8_t *out;
  uint64_t cap;
  uint64_t *tok_off;
  uint32_t *len;      // [n] byte length of each token
  uint32_t *part;     // [blocks] bytes per block of DEC_TILE tokens
  DecStatus *st;
};

// offset << 8 | length of an id's bytes in the decode blob, or 0 (bad id)
__device__ __forceinline__ uint64_t dec_entry(const DevTables &T, int32_t id) {
  if (id >= 0 && uint32_t(id) < T.dec_n) {
    const uint64_t e = T.dec[id];
    if (e) return e;
  }
  if (id < 0) return 0;
  // specials, sorted by id
  uint32_t lo = 0, hi = T.n_sp;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (T.dsp[2 * mid] < uint64_t(id)) lo = mid + 1;
    else hi = mid;
  }
  return (lo < T.n_sp && T.dsp[2 * lo] == uint64_t(id)) ? T.dsp[2 * lo + 1] : 0ull;
}

__device__ __forceinline__ uint32_t dec_block_excl_scan(uint32_t v, uint32_t *sh, uint32_t &total) {
  const uint32_t lane = threadIdx.x & 63, wv = threadIdx.x / 64;
  const uint32_t incl = wave_incl_sum(v, int(lane));
  if (lane == 63) sh[wv] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (uint32_t q = 0; q < DEC_BLOCK / 64; ++q) {
    before += q < wv ? sh[q] : 0u;
    all += sh[q];
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

__global__ void k_dec_init(DecArgs a) {
  if (threadIdx.x == 0) {
    a.st->first_bad = ~0ull;
    a.st->total = 0;
    a.st->complete = 0;
  }
}

// lengths, the first bad id, and the bytes of every block of DEC_TILE tokens
__global__ void __launch_bounds__(DEC_BLOCK) k_dec_len(DecArgs a) {
  __shared__ uint32_t sh[DEC_BLOCK / 64];
  const uint64_t b0 = uint64_t(blockIdx.x) * DEC_TILE;
  uint32_t sum = 0;
  for (uint32_t k = 0; k < DEC_ITEMS; ++k) {
    const uint64_t i = b0 + uint64_t(k) * DEC_BLOCK + threadIdx.x;  // coalesced
    if (i < a.n) {
      const uint64_t e = dec_entry(a.T, a.ids[i]);
      if (!e) atomicMin(&a.st->first_bad, static_cast<unsigned long long>(i));
      const uint32_t l = uint32_t(e & 0xFFu);
      a.len[i] = l;
      sum += l;
    }
  }
  uint32_t total;
  (void)dec_block_excl_scan(sum, sh, total);
  if (threadIdx.x == 0) a.part[blockIdx.x] = total;
}

// offsets (base from the blocks before, scan inside the block), then the
// bytes of every token when the output fits and every id is good
__global__ void __launch_bounds__(DEC_BLOCK) k_dec_copy(DecArgs a) {
  __shared__ uint32_t sh[DEC_BLOCK / 64];
  const uint64_t b0 = uint64_t(blockIdx.x) * DEC_TILE;
  const uint32_t nblk = uint32_t((a.n + DEC_TILE - 1) / DEC_TILE);
  uint64_t before = 0, every = 0;
  for (uint32_t q = threadIdx.x; q < nblk; q += DEC_BLOCK) {
    const uint32_t t = a.part[q];
    before += q < blockIdx.x ? t : 0u;
    every += t;
  }
  // (64-bit block sums: wave sums of the two halves)
  __shared__ unsigned long long s_sum[2][DEC_BLOCK / 64];
  {
    unsigned long long x = before, y = every;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      x += __shfl_xor(x, d, 64);
      y += __shfl_xor(y, d, 64);
    }
    if ((threadIdx.x & 63) == 0) {
      s_sum[0][threadIdx.x / 64] = x;
      s_sum[1][threadIdx.x / 64] = y;
    }
  }
  __syncthreads();
  uint64_t base = 0, total = 0;
#pragma unroll
  for (uint32_t q = 0; q < DEC_BLOCK / 64; ++q) {
    base += s_sum[0][q];
    total += s_sum[1][q];
  }
  const bool write = total <= a.cap && a.st->first_bad == ~0ull;
  // each thread: DEC_ITEMS consecutive tokens
  uint32_t l[DEC_ITEMS];
  uint32_t sum = 0;
#pragma unroll
  for (uint32_t k = 0; k < DEC_ITEMS; ++k) {
    const uint64_t i = b0 + uint64_t(threadIdx.x) * DEC_ITEMS + k;
    l[k] = i < a.n ? a.len[i] : 0u;
    sum += l[k];
  }
  uint32_t blk;
  uint64_t off = base + dec_block_excl_scan(sum, sh, blk);
#pragma unroll
  for (uint32_t k = 0; k < DEC_ITEMS; ++k) {
    const uint64_t i = b0 + uint64_t(threadIdx.x) * DEC_ITEMS + k;
    if (i < a.n) {
      if (a.tok_off) a.tok_off[i] = off;
      if (write) {
        const uint64_t e = dec_entry(a.T, a.ids[i]);
        const uint8_t *src = a.T.dblob + (e >> 8);
        for (uint32_t j = 0; j < l[k]; ++j) a.out[off + j] = src[j];
      }
    }
    off += l[k];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) a.st->total = total;
}

// The output length without a trailing partial character: when the last k
// bytes (k <= 3) are a proper prefix of a well-formed UTF-8 sequence (the
// Unicode standard's table of well-formed byte sequences: lead C2-DF, E0-EF
// or F0-F4, the second byte's range set by the lead), they are held back.
__global__ void k_dec_tail(DecArgs a) {
  if (threadIdx.x != 0) return;
  const uint64_t total = a.st->total;
  uint64_t complete = total;
  if (total <= a.cap && a.st->first_bad == ~0ull) {
    for (uint64_t k = 1; k <= 3 && k <= total; ++k) {
      const uint32_t b = a.out[total - k];
      if ((b & 0xC0u) == 0x80u) continue;
      // b is the last byte that is not a continuation byte
      const uint32_t need = (b >= 0xC2 && b <= 0xDF) ? 2u : (b >= 0xE0 && b <= 0xEF) ? 3u
                          : (b >= 0xF0 && b <= 0xF4) ? 4u : 0u;
      if (need > k) {
        bool ok = true;
        if (k >= 2) {
          const uint32_t s = a.out[total - k + 1];
          const uint32_t lo = b == 0xE0 ? 0xA0u : b == 0xF0 ? 0x90u : 0x80u;
          const uint32_t hi = b == 0xED ? 0x9Fu : b == 0xF4 ? 0x8Fu : 0xBFu;
          ok = s >= lo && s <= hi;
        }
        if (ok) complete = total - k;
      }
      break;
    }
  }
  a.st->complete = complete;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

struct DecLayout {
  uint64_t status, len, part, total;
};
DecLayout dec_layout(uint64_t n) {
  DecLayout L{};
  uint64_t o = 0;
  L.status = o; o = align256(o + sizeof(DecStatus));
  L.len = o; o = align256(o + 4 * (n + 1));
  L.part = o; o = align256(o + 4 * (n / DEC_TILE + 2));
  L.total = o;
  return L;
}

}  // namespace
}  // namespace bbpe

using namespace bbpe;

extern "C" {

int bbpe_decode_workspace_bytes(const bbpe_tokenizer *t, uint64_t n_ids, uint64_t *out_bytes) {
  if (!t || !out_bytes) return BBPE_E_INVALID_ARG;
  *out_bytes = dec_layout(n_ids).total;
  return BBPE_OK;
}

int bbpe_decode_device(bbpe_tokenizer *t, const int32_t *d_ids, uint64_t n_ids, uint8_t *d_out,
                       uint64_t out_capacity, uint64_t *d_tok_off, void *d_ws, uint64_t ws_bytes,
                       uint64_t *out_len, uint64_t *complete_len, void *stream) {
  if (!t || !out_len || (n_ids && !d_ids) || (out_capacity && !d_out)) return BBPE_E_INVALID_ARG;
  if (!t->d_image) return BBPE_E_STATE;
  const DecLayout L = dec_layout(n_ids);
  if (!d_ws || ws_bytes < L.total || (reinterpret_cast<uintptr_t>(d_ws) & 255)) return BBPE_E_WORKSPACE;
  uint8_t *w = static_cast<uint8_t *>(d_ws);
  DecArgs a{};
  a.T = t->dev;
  a.ids = d_ids;
  a.n = n_ids;
  a.out = d_out;
  a.cap = out_capacity;
  a.tok_off = d_tok_off;
  a.st = reinterpret_cast<DecStatus *>(w + L.status);
  a.len = reinterpret_cast<uint32_t *>(w + L.len);
  a.part = reinterpret_cast<uint32_t *>(w + L.part);
  Launcher go{t, reinterpret_cast<hipStream_t>(stream)};
  go("k_dec_init", k_dec_init, dim3(1), dim3(64), a);
  if (n_ids) {
    const uint32_t nb = uint32_t((n_ids + DEC_TILE - 1) / DEC_TILE);
    go("k_dec_len", k_dec_len, dim3(nb), dim3(DEC_BLOCK), a);
    go("k_dec_copy", k_dec_copy, dim3(nb), dim3(DEC_BLOCK), a);
    go("k_dec_tail", k_dec_tail, dim3(1), dim3(64), a);
  }
  HIP_OK(hipGetLastError());
  DecStatus h{};
  HIP_OK(hipMemcpyAsync(&h, a.st, sizeof(DecStatus), hipMemcpyDeviceToHost, go.st));
  HIP_OK(hipStreamSynchronize(go.st));
  go.collect();
  if (h.first_bad != ~0ull) {
    *out_len = h.first_bad;
    return BBPE_E_BAD_ID;
  }
  *out_len = h.total;
  if (complete_len) *complete_len = h.complete;
  return h.total > out_capacity ? BBPE_E_CAPACITY : BBPE_OK;
}

}  // extern "C"
