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
  uint64_t *tile_fn;                // [T] split transfer functions
  uint32_t *tile_carry;             // [T] split state entering each tile
  uint32_t *tile_np;                // [T+1] pieces per tile, then their exclusive scan
  uint32_t *piece_start;            // [P+1]
  uint32_t *piece_cnt;              // [P] ids per unit
  uint32_t *piece_off;              // [P+1] exclusive scan of the ids per unit
  int32_t *tmp_ids;                 // [N] ids of each piece, at the piece's byte offset
  uint32_t *scan_part;              // [N/4096+2] partial sums of the piece scan
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

// threads per k_probe block (units per block and pass)
constexpr uint32_t PROBE_BLOCK = 512;
// Texts of at most FUSE_TILES tiles skip the one-workgroup tile scans of the
// split functions and of the unit counts: every block of k_split / k_pieces
// folds the tiles before (and, for the lookahead, after) it itself.
constexpr uint32_t FUSE_TILES = 2048;
constexpr uint64_t PROBE_SMALL = 1u << 20;  // texts below this: one unit per probe thread

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
  int32_t *ids;
  uint64_t ids_cap;
  int64_t *id_off;
  WsPtrs ws;
};

__global__ void k_count(EncodeArgs a);
__global__ void k_scan_chars(EncodeArgs a);
__global__ void k_spans(EncodeArgs a);
__global__ void k_split_agg(EncodeArgs a);
__global__ void k_scan_split(EncodeArgs a);
__global__ void k_split(EncodeArgs a);
__global__ void k_split_agg_o200k(EncodeArgs a);
__global__ void k_scan_split_o200k(EncodeArgs a);
__global__ void k_split_o200k(EncodeArgs a);
__global__ void k_scan_tiles_np(EncodeArgs a);
__global__ void k_pieces(EncodeArgs a);
__global__ void k_probe(EncodeArgs a);
__global__ void k_probe1(EncodeArgs a);
__global__ void k_merge(EncodeArgs a);
__global__ void k_merge_long(EncodeArgs a);
__global__ void k_merge_group(EncodeArgs a);
__global__ void k_scan_reduce(EncodeArgs a);
__global__ void k_scan_down(EncodeArgs a);
__global__ void k_assemble(EncodeArgs a);

}  // namespace bbpe
