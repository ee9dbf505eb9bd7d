// Host planner of the encode path: table upload, workspace layout and the
// kernel sequence of bbpe_encode_segments / bbpe_pretokenize_segments.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/bbpe.h"
#include "bbpe_internal.h"
#include "bbpe_kernels.h"
#include "bbpe_launch.h"
#include "bbpe_tokenizer.h"

using namespace bbpe;

// Device scratch of bbpe_encode_segments_noalloc: the workspace of that
// entry point, a file-scope array of BBPE_NOALLOC_SCRATCH_BYTES bytes.  Each
// GPU the library runs on holds its own copy until the process ends.  Host
// code never uses this name as an address: the device address of each
// GPU's copy comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) uint8_t scratch[BBPE_NOALLOC_SCRATCH_BYTES];

namespace {

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

struct WsLayout {
  uint64_t status, tile_nchar, tile_err, tile_bad, tile_lastchg, tile_charbase, tile_chgcarry, seg_local, seg_charstart,
      ss, spst, spc, ps, tile_sp_eout, tile_sp_unres, tile_fn, tile_carry, tile_np, piece_start, piece_cnt,
      tmp_ids, uid, owner, scan_state, lst[ML_COUNT], lrank, lpart, lnl, lnr, lbits, lsel, leqm, lmin, ldirty, wslow, wseg, wseg_at, total;
  uint64_t n_words;
  uint32_t n_tiles;
  uint32_t owner_slots;
};

// Word-cache slots for a text of n bytes: a power of two of at least n/4
// (at most one unit per two bytes, and far fewer distinct ones, so that
// few byte strings share a slot), 2^12..2^23.
uint32_t owner_slots_for(uint64_t n) {
  uint64_t want = std::max<uint64_t>(n / 4, uint64_t(1) << 12);
  uint32_t s = 1u << 12;
  while (s < want && s < (1u << 23)) s <<= 1;
  return s;
}

WsLayout layout_for(uint64_t n, uint32_t n_seg) {
  WsLayout L{};
  const uint64_t W = (n + 63) / 64;
  const uint64_t T = (W + TILE_WORDS - 1) / TILE_WORDS;
  L.n_words = W;
  L.n_tiles = uint32_t(T);
  uint64_t o = 0;
  auto take = [&](uint64_t &field, uint64_t bytes) {
    field = o;
    o = align256(o + bytes);
  };
  take(L.status, sizeof(Status));
  take(L.tile_nchar, 4 * (T + 1));
  take(L.tile_err, 8 * (T + 1));
  take(L.tile_bad, 4 * (T + 1));
  take(L.tile_lastchg, 4 * (T + 1));
  take(L.tile_charbase, 8 * (T + 1));
  take(L.tile_chgcarry, 8 * (T + 1));
  take(L.seg_local, 4 * (uint64_t(n_seg) + 1));
  take(L.seg_charstart, 8 * (uint64_t(n_seg) + 1));
  take(L.ss, 8 * (W + 1));
  take(L.spst, 8 * (W + 1));
  take(L.spc, 8 * (W + 1));
  take(L.ps, 8 * (W + 1));
  take(L.tile_sp_eout, 4 * (T + 1));
  take(L.tile_sp_unres, 4 * (T + 1));
  take(L.tile_fn, 8 * (T + 1));
  take(L.tile_carry, 4 * (T + 1));
  take(L.tile_np, 4 * (T + 1));
  take(L.piece_start, 4 * (n + 1));
  take(L.piece_cnt, 4 * (n + 1));
  take(L.tmp_ids, 4 * (n + 1));
  take(L.uid, 4 * (n + 1));
  L.owner_slots = owner_slots_for(n);
  take(L.owner, 4ull * L.owner_slots);
  take(L.scan_state, 8 * ((n + 1) / ASM_UNITS + 2));
  for (uint32_t k = 0; k < ML_COUNT; ++k) take(L.lst[k], 4 * (n / ML_MIN_LEN[k] + 1));
  take(L.lrank, 4 * (n + 1));
  take(L.lpart, 4 * (n + 1));
  take(L.lnl, 4 * (n + 1));
  take(L.lnr, 4 * (n + 1));
  take(L.lbits, 8 * (n / 32 + 2));
  take(L.lsel, 8 * (n / 32 + 2));
  take(L.leqm, 8 * (n / 32 + 2));
  take(L.lmin, 4 * (n / 32 + 2));
  take(L.ldirty, 4 * (n / 32 + 2));
  take(L.wslow, 8 * SLOW_WORDS * (W + 1));
  take(L.wseg, 16 * (W + 1));
  take(L.wseg_at, 4 * (W + 1));
  L.total = o;
  return L;
}

__global__ void k_init(EncodeArgs a) {
  if (threadIdx.x == 0) {
    Status *s = a.ws.status;
    s->err_pos = ~0ull;
    s->n_pieces = 0;
    s->n_ids = 0;
    for (uint32_t k = 0; k < ML_COUNT; ++k) s->n_list[k] = 0;
  s->scan_ticket = 0;
  s->scan_fail = 0;
  s->sp_fix = 0;
    s->n_chars = 0;
    s->err_seg = 0;
    // offsets must start at 0 and end at the text length (monotonicity is
    // checked by k_count, or k_check_offsets for an empty text); every later
    // kernel exits when pad2 is set
    const bool ok = a.seg_off[0] == 0 && a.seg_off[a.n_seg] == a.n;
    s->pad2 = ok ? 0u : 1u;
  }
}

__global__ void k_check_offsets(EncodeArgs a) {
  for (uint32_t s = blockIdx.x * blockDim.x + threadIdx.x; s < a.n_seg; s += gridDim.x * blockDim.x)
    if (a.seg_off[s + 1] < a.seg_off[s]) a.ws.status->pad2 = 1u;
}

// id offsets of an empty text: all zero
__global__ void k_zero_offsets(EncodeArgs a) {
  for (uint32_t s = blockIdx.x * blockDim.x + threadIdx.x; s <= a.n_seg; s += gridDim.x * blockDim.x)
    a.id_off[s] = 0;
}

__global__ void k_copy_pieces(EncodeArgs a, uint32_t *starts, uint64_t cap, uint8_t *is_special) {
  if (a.ws.status->pad2) return;
  const uint32_t P = uint32_t(a.ws.status->n_pieces);
  if (P > cap) return;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < P; i += gridDim.x * blockDim.x) {
    const uint32_t s = a.ws.piece_start[i];
    starts[i] = s;
    if (is_special) is_special[i] = uint8_t((a.ws.spst[s >> 6] >> (s & 63)) & 1);
  }
}

__global__ void k_err_seg(EncodeArgs a) {
  const unsigned long long e = a.ws.status->err_pos;
  if (threadIdx.x == 0 && e != ~0ull) {
    uint32_t lo = 0, hi = a.n_seg;
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if (a.seg_off[mid] <= e) lo = mid + 1;
      else hi = mid;
    }
    a.ws.status->err_seg = lo > 0 ? lo - 1 : 0;
  }
}

static_assert(sizeof(Status) <= 256, "the host copy of the status block is 256 bytes");

// The last kernel of every sequence: the status block into pinned host memory.
__global__ void k_publish(EncodeArgs a, Status *host) {
  if (threadIdx.x == 0) publish_record(a, host, false);
}

// The handle's second stream and its fork/join events, created once.
int ensure_aux(bbpe_tokenizer *t) {
  if (t->aux_stream) return BBPE_OK;
  hipStream_t s = nullptr;
  hipEvent_t f = nullptr, j = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return BBPE_E_HIP;
  if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
    if (f) (void)hipEventDestroy(f);
    (void)hipStreamDestroy(s);
    return BBPE_E_HIP;
  }
  t->aux_stream = s;
  t->ev_fork = f;
  t->ev_join = j;
  return BBPE_OK;
}

// Validates arguments and carves the workspace.
int prepare(bbpe_tokenizer *t, const uint8_t *d_text, uint64_t n, const uint64_t *d_seg_off,
            const uint8_t *d_allow, uint32_t n_seg, uint32_t flags, void *d_ws, uint64_t ws_bytes,
            EncodeArgs &a, WsLayout &L) {
  if (!t || !d_seg_off || (n_seg && !d_allow)) return BBPE_E_INVALID_ARG;
  if (n && (!d_text || (reinterpret_cast<uintptr_t>(d_text) & 15))) return BBPE_E_INVALID_ARG;
  if (n >= (uint64_t(1) << 32) - 64 ||
      (flags & ~uint32_t(BBPE_TIKTOKEN_SAFE | BBPE_COUNT_ONLY | BBPE_KEEP_WORD_CACHE)))
    return BBPE_E_INVALID_ARG;
  if (n_seg == 0 && n != 0) return BBPE_E_INVALID_ARG;
  if (!t->d_image || !t->host_status) return BBPE_E_STATE;
  L = layout_for(n, n_seg);
  if (!d_ws || ws_bytes < L.total || (reinterpret_cast<uintptr_t>(d_ws) & 255)) return BBPE_E_WORKSPACE;
  uint8_t *w = static_cast<uint8_t *>(d_ws);
  a = EncodeArgs{};
  a.T = t->dev;
  a.text = d_text;
  a.n = n;
  a.seg_off = d_seg_off;
  a.allow = d_allow;
  a.n_seg = n_seg;
  a.flags = flags;
  a.n_words = L.n_words;
  a.n_tiles = L.n_tiles;
  a.ws.status = reinterpret_cast<Status *>(w + L.status);
  a.ws.tile_nchar = reinterpret_cast<uint32_t *>(w + L.tile_nchar);
  a.ws.tile_err = reinterpret_cast<unsigned long long *>(w + L.tile_err);
  a.ws.tile_bad = reinterpret_cast<uint32_t *>(w + L.tile_bad);
  a.ws.tile_lastchg = reinterpret_cast<int32_t *>(w + L.tile_lastchg);
  a.ws.tile_charbase = reinterpret_cast<unsigned long long *>(w + L.tile_charbase);
  a.ws.tile_chgcarry = reinterpret_cast<long long *>(w + L.tile_chgcarry);
  a.ws.seg_local = reinterpret_cast<uint32_t *>(w + L.seg_local);
  a.ws.seg_charstart = reinterpret_cast<unsigned long long *>(w + L.seg_charstart);
  a.ws.ss = reinterpret_cast<uint64_t *>(w + L.ss);
  a.ws.spst = reinterpret_cast<uint64_t *>(w + L.spst);
  a.ws.spc = reinterpret_cast<uint64_t *>(w + L.spc);
  a.ws.ps = reinterpret_cast<uint64_t *>(w + L.ps);
  a.ws.tile_sp_eout = reinterpret_cast<uint32_t *>(w + L.tile_sp_eout);
  a.ws.tile_sp_unres = reinterpret_cast<uint32_t *>(w + L.tile_sp_unres);
  a.ws.tile_fn = reinterpret_cast<uint64_t *>(w + L.tile_fn);
  a.ws.tile_carry = reinterpret_cast<uint32_t *>(w + L.tile_carry);
  a.ws.tile_np = reinterpret_cast<uint32_t *>(w + L.tile_np);
  a.ws.piece_start = reinterpret_cast<uint32_t *>(w + L.piece_start);
  a.ws.piece_cnt = reinterpret_cast<uint32_t *>(w + L.piece_cnt);
  a.ws.tmp_ids = reinterpret_cast<int32_t *>(w + L.tmp_ids);
  a.ws.uid = reinterpret_cast<int32_t *>(w + L.uid);
  a.ws.owner = reinterpret_cast<uint32_t *>(w + L.owner);
  a.owner_mask = L.owner_slots - 1;
  a.word_cache = n >= WORD_CACHE_MIN ? 1u : 0u;
  a.ws.scan_state = reinterpret_cast<unsigned long long *>(w + L.scan_state);
  for (uint32_t k = 0; k < ML_COUNT; ++k) a.ws.lst[k] = reinterpret_cast<uint32_t *>(w + L.lst[k]);
  a.ws.lrank = reinterpret_cast<int32_t *>(w + L.lrank);
  a.ws.lpart = reinterpret_cast<int32_t *>(w + L.lpart);
  a.ws.lnl = reinterpret_cast<int32_t *>(w + L.lnl);
  a.ws.lnr = reinterpret_cast<int32_t *>(w + L.lnr);
  a.ws.lbits = reinterpret_cast<unsigned long long *>(w + L.lbits);
  a.ws.lsel = reinterpret_cast<unsigned long long *>(w + L.lsel);
  a.ws.leqm = reinterpret_cast<unsigned long long *>(w + L.leqm);
  a.ws.lmin = reinterpret_cast<int32_t *>(w + L.lmin);
  a.ws.ldirty = reinterpret_cast<uint32_t *>(w + L.ldirty);
  a.ws.wslow = reinterpret_cast<uint64_t *>(w + L.wslow);
  a.ws.wseg = reinterpret_cast<uint64_t *>(w + L.wseg);
  a.ws.wseg_at = reinterpret_cast<uint32_t *>(w + L.wseg_at);
  return BBPE_OK;
}

// Steps up to the ordered list of piece starts.
template <typename Go>
void launch_front(Go &go, const EncodeArgs &a, const WsLayout &L) {
  // (a non-empty text has its status initialised by k_scan_chars, from the
  // per-tile results of k_count, which reads no status)
  if (a.n == 0) {
    go("k_init", k_init, dim3(1), dim3(64), a);
    if (a.n_seg)
      go("k_check_offsets", k_check_offsets, dim3(std::min<uint32_t>(1024, (a.n_seg + 255) / 256)),
         dim3(256), a);
    return;
  }
  const uint32_t T = L.n_tiles;
  go("k_count", k_count, dim3(T), dim3(64), a);
  if (T > FUSE_TILES) go("k_scan_chars", k_scan_chars, dim3(1), dim3(1024), a);
  go("k_spans", k_spans, dim3(T), dim3(64), a);
  if (a.T.sp_overlap) {
    go("k_specials", k_specials, dim3(T), dim3(64), a);
    go("k_specials_fix", k_specials_fix, dim3(1), dim3(64), a);
  }
  if (a.T.grammar == BBPE_GRAMMAR_O200K_STYLE) {
    go("k_split_agg_o200k", k_split_agg_o200k, dim3(T), dim3(64), a);
    if (T > FUSE_TILES) go("k_scan_split_o200k", k_scan_split_o200k, dim3(1), dim3(1024), a);
    go("k_split_o200k", k_split_o200k, dim3(T), dim3(64), a);
  } else {
    go("k_split_agg", k_split_agg, dim3(T), dim3(64), a);
    if (T > FUSE_TILES) go("k_scan_split", k_scan_split, dim3(1), dim3(1024), a);
    go("k_split", k_split, dim3(T), dim3(64), a);
  }
  if (T > FUSE_TILES) go("k_scan_tiles_np", k_scan_tiles_np, dim3(1), dim3(1024), a);
  go("k_pieces", k_pieces, dim3(T), dim3(64), a);
}

// Publishes the status block to the host (k_publish, the sequence's last
// kernel) unless the sequence already did.
template <typename Go>
void publish(bbpe_tokenizer *t, Go &go, const EncodeArgs &a) {
  go("k_publish", k_publish, dim3(1), dim3(64), a, static_cast<Status *>(t->host_status_dev));
}

// Clears the error fields of the host record before a call, unless calls
// enqueued without a wait are outstanding: their errors stay for the wait.
void clear_record(bbpe_tokenizer *t) {
  if (t->inflight) return;
  volatile Status *h = static_cast<volatile Status *>(t->host_status);
  h->err_pos = ~0ull;
  h->err_seg = 0u;
  h->pad2 = 0u;
  h->scan_fail = 0u;
  h->over_cap = 0u;
}

// While asynchronous encodes are outstanding, every call of the handle must
// use their stream (a wait on it then covers them all).
int check_pipeline(const bbpe_tokenizer *t, void *stream) {
  return t->inflight && stream != t->async_stream ? BBPE_E_INVALID_ARG : BBPE_OK;
}

// The first error the record holds: bad offsets, a scan that gave up
// waiting, invalid UTF-8 (its place kept for bbpe_error_detail), ids beyond
// a capacity.
int record_error(const bbpe_tokenizer *t, const Status &h) {
  if (h.pad2) return BBPE_E_INVALID_ARG;
  if (h.scan_fail) return BBPE_E_HIP;
  if (h.err_pos != ~0ull) {
    set_last_utf8_error(t, h.err_seg, h.err_pos);
    return BBPE_E_UTF8;
  }
  if (h.over_cap) return BBPE_E_CAPACITY;
  return BBPE_OK;
}

// Waits for the call (its one host synchronisation) and reads the status
// block that its last kernel wrote; this also settles every asynchronous
// call before it.
int finish(bbpe_tokenizer *t, Launcher &go, Status &h) {
  const hipError_t e0 = hipGetLastError();
  const hipError_t e1 = hipStreamSynchronize(go.st);
  t->inflight = 0;
  if (e0 != hipSuccess || e1 != hipSuccess) return BBPE_E_HIP;
  go.collect();
  memcpy(&h, t->host_status, sizeof(Status));
  return record_error(t, h);
}

// The encode kernels of `a` on go.st, and with fork the group and long
// tiers on the handle's second stream beside the short tier (joined back
// before the scan), ending with k_publish.
template <typename Go>
int enqueue_encode(bbpe_tokenizer *t, Go &go, const EncodeArgs &a, const WsLayout &L,
                   bool fork) {
  const uint64_t n = a.n;
  launch_front(go, a, L);
  const uint32_t seg_grid = std::min<uint32_t>(1024, (a.n_seg + 256) / 256);
  if (n == 0) {
    go("k_zero_offsets", k_zero_offsets, dim3(seg_grid), dim3(256), a);
  } else {
    if (n < PROBE_SMALL) {
      const uint32_t probe_grid = uint32_t((n + 2047) / 2048);
      go("k_probe", a.wcache ? k_probe1_wc : k_probe1, dim3(probe_grid), dim3(PROBE_BLOCK), a);
    } else if (n < PROBE_MID || a.wcache) {
      const uint32_t probe_grid = uint32_t(std::min<uint64_t>((n + 8191) / 8192, 8192));
      go("k_probe", a.wcache ? k_probe_wc : k_probe, dim3(probe_grid), dim3(PROBE_BLOCK), a);
    } else {
      const uint32_t probe_grid = uint32_t(std::min<uint64_t>((n + 4095) / 4096, 8192));
      go("k_probe", k_probe2, dim3(probe_grid), dim3(PROBE_BLOCK), a);
    }
    // (grid-stride kernels: their units are few, and idle waves of the
    // second stream take dispatch slots from the short tier.)
    const uint32_t wide_grid = uint32_t(std::min<uint64_t>(n / 17 + 1, 4096));
    const uint32_t long_grid = uint32_t(std::min<uint64_t>(n / 513 + 1, 64));
    const uint32_t merge_grid = uint32_t(std::min<uint64_t>((n + 255) / 256, 8192));
    // (the kept word cache has kernels of its own, so that the others carry
    // none of its code)
    auto *const merge_k = a.word_cache ? (a.wcache ? k_merge_elect_wc : k_merge_elect)
                                       : (a.wcache ? k_merge_wc : k_merge);
    auto *const wide_k = a.wcache ? k_merge_wide_wc : (a.word_cache ? k_merge_wide : k_merge_wide_few32);
    if (fork) {
      // the units of 17-512 bytes (few, long dependent chains) run on the
      // second stream beside the rest of the short tier; the long tier
      // follows the short tier on the caller's stream (a long-tier
      // workgroup needs a whole CU's LDS, which the short tier's waves hold
      // until they drain)
      // (which branch is enqueued first matters for the graph: its first
      // kernel starts about 5 us after the fork, the other's about 10.
      // Below WORD_CACHE_MIN bytes the short tier comes first, and the
      // group tier, short there, runs beside it followed by the long tier;
      // from it the group tier is the longest chain and comes first, and
      // the long tier follows the short tier.)
      int rc = go.record(0);
      if (!a.word_cache) go("k_merge", merge_k, dim3(merge_grid), dim3(64), a);
      go.use_aux();
      if (!rc) rc = go.wait(0);
      go("k_merge_wide", wide_k, dim3(wide_grid), dim3(64), a);
      if (!a.word_cache) go("k_merge_long", k_merge_long, dim3(long_grid), dim3(1024), a);
      if (!rc) rc = go.record(1);
      go.use_main();
      if (a.word_cache) {
        go("k_merge", merge_k, dim3(merge_grid), dim3(64), a);
        go("k_merge_long", k_merge_long, dim3(long_grid), dim3(1024), a);
      }
      if (!rc) rc = go.wait(1);
      if (rc) return rc;
    } else {
      go("k_merge_wide", wide_k, dim3(wide_grid), dim3(64), a);
      go("k_merge", merge_k, dim3(merge_grid), dim3(64), a);
      go("k_merge_long", k_merge_long, dim3(long_grid), dim3(1024), a);
    }
    // at most one scan tile per ASM_UNITS bytes (the unit count is at most
    // n); the single pass takes its tiles from a ticket counter on a grid of
    // at most ASM_GRID workgroups, the three-phase path one tile per
    // workgroup; the last tile publishes the status block
    const uint32_t agrid = uint32_t((n + 1 + ASM_UNITS - 1) / ASM_UNITS);
    const int single = n <= ASM_SINGLE_MAX ? 1 : 0;
    if (!single) {
      go("k_scan_sums", k_scan_sums, dim3(agrid), dim3(1024), a);
      go("k_scan_bases", k_scan_bases, dim3(1), dim3(1024), a);
    }
    if (single)
      go("k_assemble", k_assemble, dim3(std::min(agrid, ASM_GRID)), dim3(1024), a,
         static_cast<Status *>(t->host_status_dev));
    else
      go("k_assemble", k_assemble_based, dim3(agrid), dim3(1024), a,
         static_cast<Status *>(t->host_status_dev));
    return BBPE_OK;
  }
  publish(t, go, a);
  return BBPE_OK;
}

// What an encode's kernel sequence depends on besides the handle's tables:
// a built graph is replayed only for a call with the same values.
struct GraphKey {
  const void *image, *text, *seg_off, *allow, *ws, *ids, *id_off, *host, *wcache;
  uint64_t n, ids_cap;
  uint32_t n_seg, flags;
};

// Launches the handle's graph of this sequence on st, building it first (a
// GraphBuilder run of the same sequence) when the last one was built with
// other arguments.  BBPE_E_STATE when that is not possible: the caller then
// launches the kernels directly.
int run_graph(bbpe_tokenizer *t, const EncodeArgs &a, const WsLayout &L, hipStream_t st) {
  GraphKey k;
  memset(&k, 0, sizeof k);
  k.image = t->d_image;
  k.text = a.text;
  k.seg_off = a.seg_off;
  k.allow = a.allow;
  k.ws = a.ws.status;
  k.ids = a.ids;
  k.id_off = a.id_off;
  k.host = t->host_status_dev;
  k.wcache = a.wcache;
  k.n = a.n;
  k.ids_cap = a.ids_cap;
  k.n_seg = a.n_seg;
  k.flags = a.flags;
  const uint8_t *kb = reinterpret_cast<const uint8_t *>(&k);
  const bool hit = t->graph_exec && t->graph_key.size() == sizeof k &&
                   memcmp(t->graph_key.data(), kb, sizeof k) == 0;
  if (!hit) {
    if (t->graph_exec) {
      if (t->inflight) HIP_OK(hipStreamSynchronize(st));  // (replays of it may still run)
      (void)hipGraphExecDestroy(static_cast<hipGraphExec_t>(t->graph_exec));
      t->graph_exec = nullptr;
      t->graph_key.clear();
    }
    GraphBuilder gb;
    if (hipGraphCreate(&gb.g, 0) != hipSuccess) return BBPE_E_STATE;
    const int rc = enqueue_encode(t, gb, a, L, true);
    hipGraphExec_t x = nullptr;
    const bool ok = !rc && !gb.err &&
                    hipGraphInstantiate(&x, gb.g, nullptr, nullptr, 0) == hipSuccess && x;
    (void)hipGraphDestroy(gb.g);
    if (!ok) {
      (void)hipGetLastError();
      return BBPE_E_STATE;
    }
    t->graph_exec = x;
    t->graph_key.assign(kb, kb + sizeof k);
  }
  HIP_OK(hipGraphLaunch(static_cast<hipGraphExec_t>(t->graph_exec), st));
  return BBPE_OK;
}

// The encode of the encode entry points.  fork: the second stream beside
// the short tier (its stream and events created on first use), and the
// whole sequence launched as one HIP graph, built once and replayed while
// the arguments stay the same (a replay saves the host the time of
// launching a dozen kernels and events one by one); otherwise every kernel
// is launched on the caller's stream, and no stream, event, graph or memory
// is created.  async: return once the work is enqueued (n_ids unused).
int encode_impl(bbpe_tokenizer *t, const uint8_t *d_text, uint64_t n, const uint64_t *d_seg_off,
                const uint8_t *d_allow, uint32_t n_seg, uint32_t flags, void *d_ws,
                uint64_t ws_bytes, int32_t *d_ids, uint64_t ids_cap, int64_t *d_id_off,
                uint64_t *n_ids, void *stream, bool fork, bool async = false) {
  const bool count_only = (flags & BBPE_COUNT_ONLY) != 0;
  if (count_only) ids_cap = 0;  // k_assemble then copies no ids
  int rc = check_pipeline(t, stream);
  if (rc) return rc;
  EncodeArgs a;
  WsLayout L;
  rc = prepare(t, d_text, n, d_seg_off, d_allow, n_seg, flags, d_ws, ws_bytes, a, L);
  if (rc) return rc;
  a.ids = d_ids;
  a.ids_cap = ids_cap;
  a.id_off = d_id_off;
  a.merge_units = 1;
  const bool keep = (flags & BBPE_KEEP_WORD_CACHE) != 0;
  if (keep) {
    if (!fork) return BBPE_E_INVALID_ARG;  // the no-alloc entry point keeps no cache
    if (!t->wcache) {
      void *p = nullptr;
      const uint64_t bytes = uint64_t(BBPE_WORD_CACHE_ENTRIES) * WC_ENTRY_BYTES;
      HIP_OK(hipMalloc(&p, bytes));
      if (hipMemset(p, 0, bytes) != hipSuccess) {
        (void)hipFree(p);
        return BBPE_E_HIP;
      }
      t->wcache = p;
    }
    a.wcache = static_cast<uint32_t *>(t->wcache);
    a.wc_mask = BBPE_WORD_CACHE_ENTRIES - 1;
  }
  if (fork) {
    rc = ensure_aux(t);
    if (rc) return rc;
  }
  Launcher go{t, reinterpret_cast<hipStream_t>(stream)};
  go.allow_timing = fork;
  // (the previous call has completed, its stream synchronised, unless it
  // was enqueued without a wait on this same stream)
  clear_record(t);
  bool done = false;
  if (fork && !t->timing && !t->graph_broken) {
    rc = run_graph(t, a, L, go.st);
    if (rc == BBPE_E_STATE) t->graph_broken = true;
    else if (rc) return rc;
    else done = true;
  }
  if (!done) {
    rc = enqueue_encode(t, go, a, L, fork);
    if (rc) return rc;
  }
  if (async) {
    ++t->inflight;
    t->async_stream = stream;
    t->async_keep = keep;
    return BBPE_OK;
  }
  Status h{};
  rc = finish(t, go, h);
  if (rc && rc != BBPE_E_CAPACITY) return rc;
  *n_ids = h.n_ids;
  if (keep) t->wc_last_hits = h.wc_hits;
  if (rc) return rc;
  if (h.n_ids > ids_cap && !count_only) return BBPE_E_CAPACITY;
  return BBPE_OK;
}

constexpr int kMaxDevices = 64;
// One no-alloc encode at a time in this process: the calls share each GPU's
// scratch array (a call on another device waits too; it is short).
std::mutex g_noalloc_mu;
void *g_scratch_addr[kMaxDevices] = {};  // device address of `scratch`, per device

// The current device's address of `scratch`, looked up once per device
// (with that device current) and kept.  Caller holds g_noalloc_mu.
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BBPE_E_HIP;
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BBPE_E_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return BBPE_OK;
}

}  // namespace

extern "C" {

int bbpe_upload_tables(bbpe_tokenizer *t, void *d_mem, uint64_t bytes, void *stream) {
  if (!t || !d_mem) return BBPE_E_INVALID_ARG;
  std::lock_guard<std::mutex> lock(t->mu);
  if (bytes < t->layout.total || (reinterpret_cast<uintptr_t>(d_mem) & 255)) return BBPE_E_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (t->inflight)  // (outstanding encodes read the old tables; the wait reports them)
    HIP_OK(hipStreamSynchronize(static_cast<hipStream_t>(t->async_stream)));
  if (t->graph_exec) {  // (built on the old table addresses)
    (void)hipGraphExecDestroy(static_cast<hipGraphExec_t>(t->graph_exec));
    t->graph_exec = nullptr;
    t->graph_key.clear();
  }
  if (!t->host_status) {
    void *h = nullptr, *d = nullptr;
    HIP_OK(hipHostMalloc(&h, 256, hipHostMallocMapped | hipHostMallocCoherent));
    if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess) {
      (void)hipHostFree(h);
      return BBPE_E_HIP;
    }
    memset(h, 0, 256);
    t->host_status = h;
    t->host_status_dev = d;
  }
  HIP_OK(hipMemcpyAsync(d_mem, t->image.data(), t->layout.total, hipMemcpyHostToDevice, st));
  HIP_OK(hipStreamSynchronize(st));
  const uint8_t *b = static_cast<const uint8_t *>(d_mem);
  const ImageLayout &L = t->layout;
  DevTables &d = t->dev;
  d.slots = reinterpret_cast<const Slot *>(b + L.slots);
  d.ext = reinterpret_cast<const uint64_t *>(b + L.ext);
  d.blob = b + L.blob;
  d.pair = reinterpret_cast<const int32_t *>(b + L.pair);
  d.atom = reinterpret_cast<const int32_t *>(b + L.atom);
  d.uni1 = reinterpret_cast<const uint16_t *>(b + L.uni1);
  d.uni2 = b + L.uni2;
  d.sp_bytes = b + L.sp_bytes;
  d.sp_off = reinterpret_cast<const uint32_t *>(b + L.sp_off);
  d.sp_id = reinterpret_cast<const int32_t *>(b + L.sp_id);
  d.inner = reinterpret_cast<const uint32_t *>(b + L.inner);
  d.mt = reinterpret_cast<const uint64_t *>(b + L.mt);
  d.k3 = reinterpret_cast<const uint32_t *>(b + L.k3);
  d.dec = reinterpret_cast<const uint64_t *>(b + L.dec);
  d.dblob = b + L.dblob;
  d.dsp = reinterpret_cast<const uint64_t *>(b + L.dsp);
  d.q4 = reinterpret_cast<const uint32_t *>(b + L.q4);
  t->d_image = b;
  return BBPE_OK;
}

int bbpe_workspace_bytes(const bbpe_tokenizer *t, uint64_t n, uint32_t n_seg, uint64_t *out) {
  if (!t || !out) return BBPE_E_INVALID_ARG;
  if (n >= (uint64_t(1) << 32) - 64) return BBPE_E_INVALID_ARG;
  *out = layout_for(n, n_seg).total;
  return BBPE_OK;
}

int bbpe_encode_segments(bbpe_tokenizer *t, const uint8_t *d_text, uint64_t n,
                         const uint64_t *d_seg_off, const uint8_t *d_allow, uint32_t n_seg,
                         uint32_t flags, void *d_ws, uint64_t ws_bytes, int32_t *d_ids,
                         uint64_t ids_cap, int64_t *d_id_off, uint64_t *n_ids, void *stream) {
  if (!t || !d_id_off || !n_ids || (ids_cap && !d_ids)) return BBPE_E_INVALID_ARG;
  std::lock_guard<std::mutex> lock(t->mu);
  return encode_impl(t, d_text, n, d_seg_off, d_allow, n_seg, flags, d_ws, ws_bytes, d_ids,
                     ids_cap, d_id_off, n_ids, stream, true);
}

int bbpe_encode_segments_async(bbpe_tokenizer *t, const uint8_t *d_text, uint64_t n,
                               const uint64_t *d_seg_off, const uint8_t *d_allow, uint32_t n_seg,
                               uint32_t flags, void *d_ws, uint64_t ws_bytes, int32_t *d_ids,
                               uint64_t ids_cap, int64_t *d_id_off, void *stream) {
  if (!t || !d_id_off || (ids_cap && !d_ids)) return BBPE_E_INVALID_ARG;
  std::lock_guard<std::mutex> lock(t->mu);
  if (t->timing) return BBPE_E_STATE;  // (per-kernel events are read at the call's end)
  return encode_impl(t, d_text, n, d_seg_off, d_allow, n_seg, flags, d_ws, ws_bytes, d_ids,
                     ids_cap, d_id_off, nullptr, stream, true, true);
}

int bbpe_encode_wait(bbpe_tokenizer *t, void *stream, uint64_t *n_ids) {
  if (!t || !n_ids) return BBPE_E_INVALID_ARG;
  std::lock_guard<std::mutex> lock(t->mu);
  if (!t->inflight) return BBPE_E_STATE;
  if (stream != t->async_stream) return BBPE_E_INVALID_ARG;
  const hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  t->inflight = 0;
  if (e != hipSuccess) return BBPE_E_HIP;
  Status h;
  memcpy(&h, t->host_status, sizeof h);
  *n_ids = h.n_ids;
  if (t->async_keep) t->wc_last_hits = h.wc_hits;
  return record_error(t, h);
}

int bbpe_encode_segments_noalloc(bbpe_tokenizer *t, const uint8_t *d_text, uint64_t n,
                                 const uint64_t *d_seg_off, const uint8_t *d_allow,
                                 uint32_t n_seg, uint32_t flags, int32_t *d_ids, uint64_t ids_cap,
                                 int64_t *d_id_off, uint64_t *n_ids, void *stream) {
  if (!t || !d_id_off || !n_ids || (ids_cap && !d_ids)) return BBPE_E_INVALID_ARG;
  if (n >= (uint64_t(1) << 32) - 64) return BBPE_E_INVALID_ARG;
  // every workspace region is written before it is read within a call, so
  // the array needs no clearing between calls
  const uint64_t need = layout_for(n, n_seg).total;
  if (need > BBPE_NOALLOC_SCRATCH_BYTES) return BBPE_E_WORKSPACE;
  std::lock_guard<std::mutex> g(g_noalloc_mu);
  void *ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc) return rc;
  std::lock_guard<std::mutex> lock(t->mu);
  return encode_impl(t, d_text, n, d_seg_off, d_allow, n_seg, flags, ws,
                     BBPE_NOALLOC_SCRATCH_BYTES, d_ids, ids_cap, d_id_off, n_ids, stream, false);
}

int bbpe_pretokenize_segments(bbpe_tokenizer *t, const uint8_t *d_text, uint64_t n,
                              const uint64_t *d_seg_off, const uint8_t *d_allow, uint32_t n_seg,
                              uint32_t flags, void *d_ws, uint64_t ws_bytes, uint32_t *d_starts,
                              uint64_t starts_cap, uint8_t *d_is_special, uint64_t *n_pieces,
                              void *stream) {
  if (!t || !n_pieces || (starts_cap && !d_starts) || (flags & BBPE_COUNT_ONLY))
    return BBPE_E_INVALID_ARG;
  std::lock_guard<std::mutex> lock(t->mu);
  int rc = check_pipeline(t, stream);
  if (rc) return rc;
  EncodeArgs a;
  WsLayout L;
  rc = prepare(t, d_text, n, d_seg_off, d_allow, n_seg, flags, d_ws, ws_bytes, a, L);
  if (rc) return rc;
  Launcher go{t, reinterpret_cast<hipStream_t>(stream)};
  clear_record(t);
  launch_front(go, a, L);
  if (n) {
    const uint32_t g = uint32_t(std::min<uint64_t>((n + 255) / 256, 4096));
    go("k_copy_pieces", k_copy_pieces, dim3(g), dim3(256), a, d_starts, starts_cap, d_is_special);
    go("k_err_seg", k_err_seg, dim3(1), dim3(64), a);
  }
  publish(t, go, a);
  Status h{};
  rc = finish(t, go, h);
  if (rc && rc != BBPE_E_CAPACITY) return rc;
  *n_pieces = h.n_pieces;
  if (rc) return rc;
  if (h.n_pieces > starts_cap) return BBPE_E_CAPACITY;
  return BBPE_OK;
}

int bbpe_set_timing(bbpe_tokenizer *t, int enable) {
  if (!t) return BBPE_E_INVALID_ARG;
  std::lock_guard<std::mutex> lock(t->mu);
  t->timing = enable != 0;
  return BBPE_OK;
}

int bbpe_timing_report(const bbpe_tokenizer *t, uint32_t idx, const char **name, double *total_ms,
                       uint64_t *launches) {
  if (!t) return BBPE_E_INVALID_ARG;
  std::lock_guard<std::mutex> lock(const_cast<bbpe_tokenizer *>(t)->mu);
  if (idx >= t->t_names.size()) return BBPE_E_INVALID_ARG;
  if (name) *name = t->t_names[idx].c_str();
  if (total_ms) *total_ms = t->t_ms[idx];
  if (launches) *launches = t->t_launches[idx];
  return BBPE_OK;
}

void bbpe_free(bbpe_tokenizer *t) {
  if (!t) return;
  if (t->inflight) (void)hipStreamSynchronize(static_cast<hipStream_t>(t->async_stream));
  for (void *e : t->t_events)
    if (e) (void)hipEventDestroy(static_cast<hipEvent_t>(e));
  if (t->graph_exec) (void)hipGraphExecDestroy(static_cast<hipGraphExec_t>(t->graph_exec));
  if (t->host_status) (void)hipHostFree(t->host_status);
  if (t->wcache) (void)hipFree(t->wcache);
  if (t->aux_stream) {
    (void)hipStreamSynchronize(static_cast<hipStream_t>(t->aux_stream));
    (void)hipEventDestroy(static_cast<hipEvent_t>(t->ev_fork));
    (void)hipEventDestroy(static_cast<hipEvent_t>(t->ev_join));
    (void)hipStreamDestroy(static_cast<hipStream_t>(t->aux_stream));
  }
  delete t;
}

int bbpe_word_cache_clear(bbpe_tokenizer *t, void *stream) {
  if (!t) return BBPE_E_INVALID_ARG;
  std::lock_guard<std::mutex> lock(t->mu);
  if (check_pipeline(t, stream)) return BBPE_E_INVALID_ARG;
  t->wc_last_hits = 0;
  if (!t->wcache) return BBPE_OK;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  HIP_OK(hipMemsetAsync(t->wcache, 0, uint64_t(BBPE_WORD_CACHE_ENTRIES) * WC_ENTRY_BYTES, st));
  HIP_OK(hipStreamSynchronize(st));
  return BBPE_OK;
}

int bbpe_word_cache_info(bbpe_tokenizer *t, uint64_t *entries, uint64_t *last_hits) {
  if (!t) return BBPE_E_INVALID_ARG;
  std::lock_guard<std::mutex> lock(t->mu);
  if (entries) *entries = t->wcache ? BBPE_WORD_CACHE_ENTRIES : 0;
  if (last_hits) *last_hits = t->wc_last_hits;
  return BBPE_OK;
}

int bbpe_timing_reset(bbpe_tokenizer *t) {
  if (!t) return BBPE_E_INVALID_ARG;
  std::lock_guard<std::mutex> lock(t->mu);
  for (auto &v : t->t_ms) v = 0.0;
  for (auto &v : t->t_launches) v = 0;
  return BBPE_OK;
}

}  // extern "C"
