// Decode on the device (gfx950): ids to bytes, each token's bytes gathered
// at its offset in the output, the offsets being the exclusive scan of the
// tokens' byte lengths (tiktoken deep-dive page, "An encoding is three
// objects": decoding concatenates the tokens' bytes; specials decode to
// their strings).  The same offsets are each token's byte offset in the text
// it was encoded from, an optional output.  The tail check reports how much
// of the output ends on a complete UTF-8 character, so that a streaming
// caller can hold the rest back (a token may end inside a character).
#include <hip/hip_runtime.h>

#include <mutex>
#include <new>

#include <algorithm>

#include "../../include/bbpe.h"
#include "bbpe_device.h"
#include "bbpe_internal.h"
#include "bbpe_launch.h"
#include "bbpe_tokenizer.h"

namespace bbpe {
namespace {

constexpr uint32_t DEC_BLOCK = 256, DEC_ITEMS = 8, DEC_TILE = DEC_BLOCK * DEC_ITEMS;
// output bytes of one tile staged in LDS (more: written straight to HBM)
constexpr uint32_t DEC_STAGE = 32768;
// up to this many tiles, every tile sums the byte counts of the tiles before
// it itself; beyond, a one-workgroup scan does it once (the per-tile sums
// grow with the square of the tile count)
constexpr uint32_t DEC_FOLD = 2048;

struct DecStatus {
  unsigned long long first_bad;  // index of the first id that is neither rank nor special, or ~0
  unsigned long long total;      // output bytes
  unsigned long long complete;   // bytes up to the end of the last complete character
                                 // (carried bytes included)
  unsigned long long tail;       // the last three bytes (carried bytes included), the
                                 // last in bits 0-7
};

struct DecArgs {
  DevTables T;
  const int32_t *ids;
  uint64_t n;
  uint8_t *out;
  uint64_t cap;
  uint64_t *tok_off;
  uint32_t *part;              // [blocks] bytes of each tile of DEC_TILE tokens
  unsigned long long *pre;     // [blocks] bytes before each tile (more than DEC_FOLD tiles)
  unsigned long long *bad;     // [blocks] first bad index of each tile, or ~0
  DecStatus *st;
  uint32_t vec_ids, vec_off;   // ids / tok_off 16-byte aligned: vector loads / stores
  uint32_t carry, n_carry;     // bytes a stream decoder held back (n_carry <= 3, the first
                               // in bits 0-7), placed just before out
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

__device__ __forceinline__ unsigned long long wave_sum64(unsigned long long v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}
__device__ __forceinline__ unsigned long long wave_min64(unsigned long long v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const unsigned long long o = __shfl_xor(v, d, 64);
    v = o < v ? o : v;
  }
  return v;
}

// Per tile: the bytes of its tokens and its first bad id (coalesced reads).
__global__ void __launch_bounds__(DEC_BLOCK) k_dec_len(DecArgs a) {
  __shared__ unsigned long long s_sum[DEC_BLOCK / 64], s_bad[DEC_BLOCK / 64];
  const uint64_t b0 = uint64_t(blockIdx.x) * DEC_TILE;
  uint32_t sum = 0;
  unsigned long long bad = ~0ull;
#pragma unroll 4
  for (uint32_t k = 0; k < DEC_ITEMS; ++k) {
    const uint64_t i = b0 + uint64_t(k) * DEC_BLOCK + threadIdx.x;
    if (i < a.n) {
      const uint64_t e = dec_entry(a.T, a.ids[i]);
      if (!e && i < bad) bad = i;
      sum += uint32_t(e & 0xFFu);
    }
  }
  const unsigned long long ws = wave_sum64(sum), wb = wave_min64(bad);
  if ((threadIdx.x & 63) == 0) {
    s_sum[threadIdx.x / 64] = ws;
    s_bad[threadIdx.x / 64] = wb;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long t = 0, m = ~0ull;
#pragma unroll
    for (uint32_t q = 0; q < DEC_BLOCK / 64; ++q) {
      t += s_sum[q];
      m = s_bad[q] < m ? s_bad[q] : m;
    }
    a.part[blockIdx.x] = uint32_t(t);
    a.bad[blockIdx.x] = m;
  }
}

// Per tile: its base (bytes of the tiles before), every token's offset (a
// block scan over runs of DEC_ITEMS consecutive tokens per thread), then its
// bytes: staged in LDS at the output's 16-byte phase and stored as aligned
// 16-byte words.  The last tile also finds the end of the last complete
// character from the last tokens' bytes.
// (more than DEC_FOLD tiles, one workgroup) bytes before every tile, the
// total and the first bad id, into pre[] and the status
__global__ void __launch_bounds__(1024) k_dec_scan(DecArgs a, uint32_t nblk) {
  __shared__ unsigned long long s_sum[2 * 16 + 1];
  __shared__ unsigned long long s_bad[16];
  const uint32_t tid = threadIdx.x;
  const uint32_t per = (nblk + 1023) / 1024;
  const uint32_t q0 = min(nblk, tid * per), q1 = min(nblk, q0 + per);
  unsigned long long sum = 0, bad = ~0ull;
  for (uint32_t q = q0; q < q1; ++q) {
    sum += a.part[q];
    bad = min(bad, a.bad[q]);
  }
  unsigned long long total;
  unsigned long long run = block_incl_scan<1024>(
      sum, 0ull, [](unsigned long long x, unsigned long long y) { return x + y; }, s_sum, total) - sum;
  for (uint32_t q = q0; q < q1; ++q) {
    a.pre[q] = run;
    run += a.part[q];
  }
  bad = wave_min64(bad);
  if ((tid & 63) == 0) s_bad[tid / 64] = bad;
  __syncthreads();
  if (tid == 0) {
    unsigned long long b = ~0ull;
    for (uint32_t w = 0; w < 16; ++w) b = min(b, s_bad[w]);
    a.st->total = total;
    a.st->first_bad = b;
  }
}

__global__ void __launch_bounds__(DEC_BLOCK) k_dec_copy(DecArgs a) {
  __shared__ unsigned long long s_a[DEC_BLOCK / 64], s_b[DEC_BLOCK / 64], s_c[DEC_BLOCK / 64];
  __shared__ uint32_t s_scan[2 * (DEC_BLOCK / 64) + 1];
  __shared__ __align__(16) uint8_t stage[DEC_STAGE + 32];
  const uint32_t nblk = gridDim.x;
  const uint32_t lane = threadIdx.x & 63, wv = threadIdx.x / 64;
  uint64_t base = 0, total = 0;
  unsigned long long first_bad = ~0ull;
  if (nblk > DEC_FOLD) {
    base = a.pre[blockIdx.x];
    total = a.st->total;
    first_bad = a.st->first_bad;
  } else {
  // base, total and the first bad id over all tiles
  unsigned long long before = 0, every = 0, bad = ~0ull;
  for (uint32_t q = threadIdx.x; q < nblk; q += DEC_BLOCK) {
    const unsigned long long t = a.part[q];
    before += q < blockIdx.x ? t : 0ull;
    every += t;
    const unsigned long long m = a.bad[q];
    bad = m < bad ? m : bad;
  }
  before = wave_sum64(before);
  every = wave_sum64(every);
  bad = wave_min64(bad);
  if (lane == 0) {
    s_a[wv] = before;
    s_b[wv] = every;
    s_c[wv] = bad;
  }
  __syncthreads();
#pragma unroll
  for (uint32_t q = 0; q < DEC_BLOCK / 64; ++q) {
    base += s_a[q];
    total += s_b[q];
    first_bad = s_c[q] < first_bad ? s_c[q] : first_bad;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.st->total = total;
    a.st->first_bad = first_bad;
  }
  }
  if (first_bad != ~0ull) return;  // (uniform over the grid)

  // this thread's DEC_ITEMS consecutive tokens
  const uint64_t i0 = uint64_t(blockIdx.x) * DEC_TILE + uint64_t(threadIdx.x) * DEC_ITEMS;
  uint64_t e[DEC_ITEMS];
  uint32_t sum = 0;
  if (a.vec_ids && i0 + DEC_ITEMS <= a.n) {
    const int4 *p = reinterpret_cast<const int4 *>(a.ids + i0);
#pragma unroll
    for (uint32_t v = 0; v < DEC_ITEMS / 4; ++v) {
      const int4 x = p[v];
      e[4 * v + 0] = dec_entry(a.T, x.x);
      e[4 * v + 1] = dec_entry(a.T, x.y);
      e[4 * v + 2] = dec_entry(a.T, x.z);
      e[4 * v + 3] = dec_entry(a.T, x.w);
    }
  } else {
#pragma unroll
    for (uint32_t k = 0; k < DEC_ITEMS; ++k)
      e[k] = i0 + k < a.n ? dec_entry(a.T, a.ids[i0 + k]) : 0ull;
  }
#pragma unroll
  for (uint32_t k = 0; k < DEC_ITEMS; ++k) sum += uint32_t(e[k] & 0xFFu);
  uint32_t blk;
  const uint32_t incl = block_incl_scan<DEC_BLOCK>(
      sum, 0u, [](uint32_t x, uint32_t y) { return x + y; }, s_scan, blk);
  const uint32_t mine = incl - sum;  // offset of this thread's first token in the tile

  if (a.tok_off) {
    uint64_t o = base + mine;
    if (a.vec_off && i0 + DEC_ITEMS <= a.n) {
      ulonglong2 *q = reinterpret_cast<ulonglong2 *>(a.tok_off + i0);
#pragma unroll
      for (uint32_t k = 0; k < DEC_ITEMS; k += 2) {
        ulonglong2 v;
        v.x = o;
        o += e[k] & 0xFFu;
        v.y = o;
        o += e[k + 1] & 0xFFu;
        q[k / 2] = v;
      }
    } else {
#pragma unroll
      for (uint32_t k = 0; k < DEC_ITEMS; ++k) {
        if (i0 + k < a.n) a.tok_off[i0 + k] = o;
        o += e[k] & 0xFFu;
      }
    }
  }

  if (total <= a.cap) {
    if (blk <= DEC_STAGE) {
      // LDS byte j <-> the output byte at address (out + base) rounded down
      // to 16, plus j
      const uint32_t phase = uint32_t((reinterpret_cast<uintptr_t>(a.out) + base) & 15);
      uint32_t o = phase + mine;
      // four tokens at a time: the first 8 bytes of each from three aligned
      // dwords of the blob (padded, so the reads stay inside it), all twelve
      // loads issued before any byte is stored; longer tokens copy the rest
#pragma unroll
      for (uint32_t k0 = 0; k0 < DEC_ITEMS; k0 += 4) {
        uint32_t wd[4][3];
#pragma unroll
        for (uint32_t c = 0; c < 4; ++c) {
          const uint32_t *q = reinterpret_cast<const uint32_t *>(a.T.dblob + ((e[k0 + c] >> 8) & ~uint64_t(3)));
          wd[c][0] = q[0];
          wd[c][1] = q[1];
          wd[c][2] = q[2];
        }
#pragma unroll
        for (uint32_t c = 0; c < 4; ++c) {
          const uint64_t ek = e[k0 + c];
          const uint32_t len = uint32_t(ek & 0xFFu), sh = uint32_t((ek >> 8) & 3u);
          const uint64_t v = uint64_t(__builtin_amdgcn_alignbyte(wd[c][1], wd[c][0], sh)) |
                             (uint64_t(__builtin_amdgcn_alignbyte(wd[c][2], wd[c][1], sh)) << 32);
          const uint32_t head = min(len, 8u);
          for (uint32_t j = 0; j < head; ++j) stage[o + j] = uint8_t(v >> (8 * j));
          const uint8_t *src = a.T.dblob + (ek >> 8);
          for (uint32_t j = 8; j < len; ++j) stage[o + j] = src[j];
          o += len;
        }
      }
      __syncthreads();
      uint8_t *dst = a.out + base - phase;
      const uint32_t end = phase + blk, nchunk = (end + 15) / 16;
      for (uint32_t c = threadIdx.x; c < nchunk; c += DEC_BLOCK) {
        const uint32_t lo = c * 16, hi = lo + 16;
        if (lo >= phase && hi <= end) {
          *reinterpret_cast<uint4 *>(dst + lo) = *reinterpret_cast<const uint4 *>(stage + lo);
        } else {
          for (uint32_t j = lo < phase ? phase : lo; j < (hi < end ? hi : end); ++j) dst[j] = stage[j];
        }
      }
    } else {
      uint64_t o = base + mine;
#pragma unroll
      for (uint32_t k = 0; k < DEC_ITEMS; ++k) {
        const uint32_t len = uint32_t(e[k] & 0xFFu);
        const uint8_t *src = a.T.dblob + (e[k] >> 8);
        for (uint32_t j = 0; j < len; ++j) a.out[o + j] = src[j];
        o += len;
      }
    }
  }

  // The output length without a trailing partial character: when the last k
  // bytes (k <= 3) are a proper prefix of a well-formed UTF-8 sequence (the
  // Unicode standard's table of well-formed byte sequences: lead C2-DF,
  // E0-EF or F0-F4, the second byte's range set by the lead), they are held
  // back.  The last bytes are read from the last tokens (each has >= 1 byte),
  // then from the carried bytes before them.  Block 0 writes the carried
  // bytes.
  if (blockIdx.x == 0 && threadIdx.x == 0 && total <= a.cap)
    for (uint32_t j = 0; j < a.n_carry; ++j) a.out[int64_t(j) - int64_t(a.n_carry)] = uint8_t(a.carry >> (8 * j));
  if (blockIdx.x == nblk - 1 && threadIdx.x == 0) {
    uint32_t tail[3] = {0, 0, 0};  // tail[k-1] = output byte total - k
    uint32_t got = 0;
    for (uint64_t t = a.n; t > 0 && got < 3; --t) {
      const uint64_t et = dec_entry(a.T, a.ids[t - 1]);
      const uint8_t *src = a.T.dblob + (et >> 8);
      for (uint32_t j = uint32_t(et & 0xFFu); j > 0 && got < 3; --j) tail[got++] = src[j - 1];
    }
    for (uint32_t j = a.n_carry; j > 0 && got < 3; --j) tail[got++] = (a.carry >> (8 * (j - 1))) & 0xFFu;
    const uint64_t all = total + a.n_carry;
    uint64_t complete = all;
    for (uint32_t k = 1; k <= got; ++k) {
      const uint32_t b = tail[k - 1];
      if ((b & 0xC0u) == 0x80u) continue;
      // b is the last byte that is not a continuation byte
      const uint32_t need = (b >= 0xC2 && b <= 0xDF) ? 2u : (b >= 0xE0 && b <= 0xEF) ? 3u
                          : (b >= 0xF0 && b <= 0xF4) ? 4u : 0u;
      if (need > k) {
        bool ok = true;
        if (k >= 2) {
          const uint32_t s = tail[k - 2];
          const uint32_t lo = b == 0xE0 ? 0xA0u : b == 0xF0 ? 0x90u : 0x80u;
          const uint32_t hi = b == 0xED ? 0x9Fu : b == 0xF4 ? 0x8Fu : 0xBFu;
          ok = s >= lo && s <= hi;
        }
        if (ok) complete = all - k;
      }
      break;
    }
    a.st->complete = complete;
    a.st->tail = tail[0] | (tail[1] << 8) | (tail[2] << 16);
  }
}

// The carried bytes alone (a stream decoder's final call with no ids).
__global__ void k_dec_carry(uint8_t *out, uint32_t carry, uint32_t n_carry) {
  for (uint32_t j = 0; j < n_carry; ++j) out[j] = uint8_t(carry >> (8 * j));
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

struct DecLayout {
  uint64_t status, part, bad, pre, total;
};
DecLayout dec_layout(uint64_t n) {
  DecLayout L{};
  const uint64_t nb = n / DEC_TILE + 2;
  uint64_t o = 0;
  L.status = o; o = align256(o + sizeof(DecStatus));
  L.part = o; o = align256(o + 4 * nb);
  L.bad = o; o = align256(o + 8 * nb);
  L.pre = o; o = align256(o + 8 * nb);
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

// d_out / out_capacity: where the ids' bytes go; n_carry carried bytes are
// written just before d_out.
static int decode_run(bbpe_tokenizer *t, const int32_t *d_ids, uint64_t n_ids, uint8_t *d_out,
                      uint64_t out_capacity, uint64_t *d_tok_off, void *d_ws, uint64_t ws_bytes,
                      void *stream, DecStatus &h, uint32_t carry = 0, uint32_t n_carry = 0) {
  if (!t->d_image) return BBPE_E_STATE;
  const DecLayout L = dec_layout(n_ids);
  if (!d_ws || ws_bytes < L.total || (reinterpret_cast<uintptr_t>(d_ws) & 255)) return BBPE_E_WORKSPACE;
  h = DecStatus{};
  h.first_bad = ~0ull;
  if (n_ids == 0) return BBPE_OK;
  if (d_tok_off && (reinterpret_cast<uintptr_t>(d_tok_off) & 7)) return BBPE_E_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(d_ids) & 3) || n_ids >= (uint64_t(1) << 40)) return BBPE_E_INVALID_ARG;
  uint8_t *w = static_cast<uint8_t *>(d_ws);
  DecArgs a{};
  a.T = t->dev;
  a.ids = d_ids;
  a.n = n_ids;
  a.out = d_out;
  a.cap = out_capacity;
  a.tok_off = d_tok_off;
  a.st = reinterpret_cast<DecStatus *>(w + L.status);
  a.part = reinterpret_cast<uint32_t *>(w + L.part);
  a.bad = reinterpret_cast<unsigned long long *>(w + L.bad);
  a.pre = reinterpret_cast<unsigned long long *>(w + L.pre);
  a.vec_ids = (reinterpret_cast<uintptr_t>(d_ids) & 15) == 0;
  a.vec_off = (reinterpret_cast<uintptr_t>(d_tok_off) & 15) == 0;
  a.carry = carry;
  a.n_carry = n_carry;
  Launcher go{t, reinterpret_cast<hipStream_t>(stream)};
  const uint32_t nb = uint32_t((n_ids + DEC_TILE - 1) / DEC_TILE);
  go("k_dec_len", k_dec_len, dim3(nb), dim3(DEC_BLOCK), a);
  if (nb > DEC_FOLD) go("k_dec_scan", k_dec_scan, dim3(1), dim3(1024), a, nb);
  go("k_dec_copy", k_dec_copy, dim3(nb), dim3(DEC_BLOCK), a);
  HIP_OK(hipGetLastError());
  HIP_OK(hipMemcpyAsync(&h, a.st, sizeof(DecStatus), hipMemcpyDeviceToHost, go.st));
  HIP_OK(hipStreamSynchronize(go.st));
  go.collect();
  return BBPE_OK;
}

int bbpe_decode_device(bbpe_tokenizer *t, const int32_t *d_ids, uint64_t n_ids, uint8_t *d_out,
                       uint64_t out_capacity, uint64_t *d_tok_off, void *d_ws, uint64_t ws_bytes,
                       uint64_t *out_len, uint64_t *complete_len, void *stream) {
  if (!t || !out_len || (n_ids && !d_ids) || (out_capacity && !d_out)) return BBPE_E_INVALID_ARG;
  std::lock_guard<std::mutex> lock(t->mu);
  DecStatus h;
  const int rc = decode_run(t, d_ids, n_ids, d_out, out_capacity, d_tok_off, d_ws, ws_bytes, stream, h);
  if (rc) return rc;
  if (h.first_bad != ~0ull) {
    *out_len = h.first_bad;
    return BBPE_E_BAD_ID;
  }
  *out_len = h.total;
  if (complete_len) *complete_len = h.complete;
  return h.total > out_capacity ? BBPE_E_CAPACITY : BBPE_OK;
}

}  // extern "C"

// A stream decoder: the bytes held back at the end of the last call.
struct bbpe_stream_decoder {
  bbpe_tokenizer *tok;
  uint32_t held, n_held;  // n_held <= 3 bytes, the first in bits 0-7
};

extern "C" {

int bbpe_stream_decoder_create(bbpe_tokenizer *tok, bbpe_stream_decoder **out) {
  if (!tok || !out) return BBPE_E_INVALID_ARG;
  *out = new (std::nothrow) bbpe_stream_decoder{tok, 0, 0};
  return *out ? BBPE_OK : BBPE_E_NOMEM;
}

int bbpe_stream_decoder_free(bbpe_stream_decoder *dec) {
  delete dec;
  return BBPE_OK;
}

int bbpe_stream_decoder_reset(bbpe_stream_decoder *dec) {
  if (!dec) return BBPE_E_INVALID_ARG;
  dec->held = dec->n_held = 0;
  return BBPE_OK;
}

int bbpe_stream_decode_device(bbpe_stream_decoder *dec, const int32_t *d_ids, uint64_t n_ids, int final,
                              uint8_t *d_out, uint64_t out_capacity, void *d_ws, uint64_t ws_bytes,
                              uint64_t *out_len, void *stream) {
  if (!dec || !out_len || (n_ids && !d_ids) || (out_capacity && !d_out)) return BBPE_E_INVALID_ARG;
  bbpe_tokenizer *t = dec->tok;
  const uint32_t nh = dec->n_held;
  if (n_ids == 0) {  // only the held bytes: emitted when final, else still held
    if (!final) {
      *out_len = 0;
      return BBPE_OK;
    }
    if (out_capacity < nh) {
      *out_len = nh;
      return BBPE_E_CAPACITY;
    }
    if (nh) {
      std::lock_guard<std::mutex> lock(t->mu);
      const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
      k_dec_carry<<<1, 1, 0, st>>>(d_out, dec->held, nh);
      HIP_OK(hipGetLastError());
      HIP_OK(hipStreamSynchronize(st));
    }
    *out_len = nh;
    dec->held = dec->n_held = 0;
    return BBPE_OK;
  }
  DecStatus h;
  {
    std::lock_guard<std::mutex> lock(t->mu);
    const uint64_t cap = out_capacity >= nh ? out_capacity - nh : 0;
    const int rc = decode_run(t, d_ids, n_ids, out_capacity >= nh ? d_out + nh : d_out, cap, nullptr, d_ws,
                              ws_bytes, stream, h, dec->held, out_capacity >= nh ? nh : 0);
    if (rc) return rc;
    if (h.first_bad != ~0ull) {
      *out_len = h.first_bad;
      return BBPE_E_BAD_ID;
    }
    if (out_capacity < nh || h.total > cap) {
      *out_len = h.total + nh;
      return BBPE_E_CAPACITY;
    }
  }
  const uint64_t all = h.total + nh;
  const uint64_t emit = final ? all : h.complete;
  const uint32_t k = uint32_t(all - emit);  // <= 3: a proper prefix of one character
  uint32_t held = 0;
  for (uint32_t j = 0; j < k; ++j) held |= ((uint32_t(h.tail) >> (8 * (k - 1 - j))) & 0xFFu) << (8 * j);
  dec->held = held;
  dec->n_held = k;
  *out_len = emit;
  return BBPE_OK;
}

int bbpe_token_offsets_device(bbpe_tokenizer *t, const int32_t *d_ids, uint64_t n_ids,
                              uint64_t *d_tok_off, void *d_ws, uint64_t ws_bytes,
                              uint64_t *total_bytes, void *stream) {
  if (!t || !total_bytes || (n_ids && (!d_ids || !d_tok_off))) return BBPE_E_INVALID_ARG;
  std::lock_guard<std::mutex> lock(t->mu);
  DecStatus h;
  const int rc = decode_run(t, d_ids, n_ids, nullptr, 0, d_tok_off, d_ws, ws_bytes, stream, h);
  if (rc) return rc;
  if (h.first_bad != ~0ull) {
    *total_bytes = h.first_bad;
    return BBPE_E_BAD_ID;
  }
  *total_bytes = h.total;
  return BBPE_OK;
}

}  // extern "C"
