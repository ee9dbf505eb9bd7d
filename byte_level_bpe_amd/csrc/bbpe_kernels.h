// Kernel arguments and entry points of the encode path (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bbpe.h"
#include "bbpe_internal.h"

namespace bbpe {

// 64-bit words of a word's stored multi-byte class record
constexpr uint32_t SLOW_WORDS = 10;

// Device workspace, carved out of the caller's buffer by the host planner.
struct WsPtrs {
  Status *status;
  uint32_t *tile_nchar;             // [T] characters per tile
  unsigned long long *tile_err;     // [T] first invalid UTF-8 byte of the tile, or ~0
  uint32_t *tile_bad;               // [T] 1: a decreasing segment offset was seen
  int32_t *tile_lastchg;            // [T] tile-local index of the last run change, or -1
  unsigned long long *tile_charbase;  // [T] index of the tile's first character
  long long *tile_chgcarry;         // [T] last run change before the tile, or -1
  uint32_t *seg_local;              // [S+1] tile-local character index of each segment start
  unsigned long long *seg_charstart;  // [S+1]
  uint64_t *ss, *spst, *spc;        // [W] span start / special start / inside special
  uint64_t *ps;                     // [W] piece starts
  uint32_t *tile_sp_eout;           // [T] (specials that can overlap) bytes of the next tile
                                    //     that the tile's last special covers
  uint32_t *tile_sp_unres;          // [T] 1: the tile's special pass is left to k_specials_fix
  uint64_t *tile_fn;                // [T] split transfer functions
  uint32_t *tile_carry;             // [T] split state entering each tile
  uint32_t *tile_np;                // [T+1] pieces per tile, then their exclusive scan
  uint32_t *piece_start;            // [P+1]
  uint32_t *piece_cnt;              // [P] ids per unit
  int32_t *tmp_ids;                 // [N] ids of each merged unit, at the unit's byte offset
  // per unit: its one id (>= 0: a special, a single byte or a key that
  // merges back to itself), UID_MERGED (its ids are at tmp_ids + its start,
  // piece_cnt of them), or UID_FOLLOW - j for a unit whose bytes equal those
  // of unit j, which merged for both (the word cache of one call)
  int32_t *uid;
  // word cache: unit index stored under a hash of each 2-16-byte unit's
  // bytes (the last store wins); [owner_mask + 1]
  uint32_t *owner;
  // per scan tile of ASM_UNITS units (k_assemble): 0 (not yet published),
  // or a flag in bits 62-63 (SCAN_AGG: the tile's own id count; SCAN_PREFIX:
  // the ids of every unit up to the tile's end) over the value
  unsigned long long *scan_state;
  uint32_t *lst[ML_COUNT];          // units to merge, by length class
  // long tier, per text position: pair rank at each part start, id of the
  // part starting there, and the two created-pair ranks of a batch merge
  int32_t *lrank, *lpart, *lnl, *lnr;
  // long tier, per 64-position block of a unit (index (s >> 5) + block):
  // part starts, selected pair starts, least pair rank, stale-minimum flag
  unsigned long long *lbits, *lsel, *leqm;
  int32_t *lmin;
  uint32_t *ldirty;
  // per text word, stored by the first front-end kernel: the multi-byte part
  // of its class masks (SLOW_WORDS each, words with a byte >= 0x80 only),
  // and its segment marks (more than one segment only)
  uint64_t *wslow;
  uint64_t *wseg;                   // [W][2]
  uint32_t *wseg_at;                // [W]
};

// units per tile of the id-count scan in k_assemble
constexpr uint32_t ASM_UNITS = 4096;
// texts up to this size scan the tiles' id counts in k_assemble itself
// (look-back between tiles); larger ones scan the tile sums apart first
constexpr uint64_t ASM_SINGLE_MAX = 6000000;
constexpr uint32_t ASM_GRID = 256;  // workgroups of the single-pass assembly at most

// threads per k_probe block (units per block and pass)
constexpr uint32_t PROBE_BLOCK = 512;
// Texts of at most FUSE_TILES tiles skip the one-workgroup tile scans of the
// split functions and of the unit counts: every block of k_split / k_pieces
// folds the tiles before (and, for the lookahead, after) it itself.
constexpr uint32_t FUSE_TILES = 4096;
constexpr uint64_t PROBE_SMALL = 1u << 20;  // texts below this: one unit per probe thread
constexpr uint64_t PROBE_MID = 1u << 23;    // texts from this: two units per probe thread
// Texts from this size on use the word cache.  Below it the short tier's
// units fit in about one generation of resident waves, so its length is
// its longest chain of merge rounds, which the cache's election only delays.
constexpr uint64_t WORD_CACHE_MIN = 8u << 20;

constexpr int32_t UID_MERGED = -1;
constexpr int32_t UID_FOLLOW = -2;  // UID_FOLLOW - j: follows unit j

constexpr uint64_t WC_ENTRY_BYTES = 128;  // one kept-word-cache entry (32 dwords)

struct EncodeArgs {
  DevTables T;
  const uint8_t *text;
  uint64_t n;
  const uint64_t *seg_off;
  const uint8_t *allow;
  uint32_t n_seg;
  uint32_t flags;
  uint64_t n_words;
  uint32_t n_tiles;
  int32_t merge_units;   // 1: cut pieces into merge units (encode); 0: pieces (pre-tokenize)
  uint32_t owner_mask;   // word-cache slots - 1 (a power of two minus one)
  uint32_t word_cache;   // 1: units of 2-16 bytes merge once per byte string (texts of at
                         //    least WORD_CACHE_MIN bytes)
  uint32_t *wcache;      // word cache kept across calls (BBPE_KEEP_WORD_CACHE), or null
                         // (WC_ENTRY_BYTES per entry)
  uint32_t wc_mask;      // its entries - 1 (a power of two minus one)
  int32_t *ids;
  uint64_t ids_cap;
  int64_t *id_off;
  WsPtrs ws;
};

// The call's status block into the host's pinned record (one thread, the
// sequence's last step).  Counts are the call's own; the error fields only
// ever go from clear to set here (the host clears them before a call when no
// other call is outstanding), so that after several calls enqueued without a
// wait the record still shows whether any of them failed: the first invalid
// UTF-8 byte met, bad offsets, ids beyond a call's capacity.
__device__ __forceinline__ void publish_record(const EncodeArgs &a, Status *host, bool ids_out) {
  const Status &d = *a.ws.status;
  host->n_pieces = d.n_pieces;
  host->n_ids = d.n_ids;
  host->n_chars = d.n_chars;
  for (uint32_t k = 0; k < ML_COUNT; ++k) host->n_list[k] = d.n_list[k];
  host->scan_ticket = d.scan_ticket;
  host->wc_hits = d.wc_hits;
  if (d.pad2) host->pad2 = d.pad2;
  if (d.err_pos != ~0ull && host->err_pos == ~0ull) {
    host->err_seg = d.err_seg;
    host->err_pos = d.err_pos;
  }
  if (ids_out && !(a.flags & BBPE_COUNT_ONLY) && d.n_ids > a.ids_cap) host->over_cap = 1u;
  __threadfence_system();
}

__global__ void k_count(EncodeArgs a);
__global__ void k_scan_chars(EncodeArgs a);
__global__ void k_spans(EncodeArgs a);
__global__ void k_specials(EncodeArgs a);
__global__ void k_specials_fix(EncodeArgs a);
__global__ void k_split_agg(EncodeArgs a);
__global__ void k_scan_split(EncodeArgs a);
__global__ void k_split(EncodeArgs a);
__global__ void k_split_agg_o200k(EncodeArgs a);
__global__ void k_scan_split_o200k(EncodeArgs a);
__global__ void k_split_o200k(EncodeArgs a);
__global__ void k_scan_tiles_np(EncodeArgs a);
__global__ void k_pieces(EncodeArgs a);
__global__ void k_probe(EncodeArgs a);
__global__ void k_probe2(EncodeArgs a);
__global__ void k_probe1(EncodeArgs a);
__global__ void k_merge(EncodeArgs a);
__global__ void k_merge_elect(EncodeArgs a);
__global__ void k_merge_elect_wc(EncodeArgs a);
__global__ void k_merge_long(EncodeArgs a);
__global__ void k_merge_wide(EncodeArgs a);
__global__ void k_merge_wide_few32(EncodeArgs a);
__global__ void k_probe_wc(EncodeArgs a);
__global__ void k_probe1_wc(EncodeArgs a);
__global__ void k_merge_wc(EncodeArgs a);
__global__ void k_merge_wide_wc(EncodeArgs a);
__global__ void k_scan_sums(EncodeArgs a);
__global__ void k_scan_bases(EncodeArgs a);
__global__ void k_assemble(EncodeArgs a, Status *host);
__global__ void k_assemble_based(EncodeArgs a, Status *host);

}  // namespace bbpe
