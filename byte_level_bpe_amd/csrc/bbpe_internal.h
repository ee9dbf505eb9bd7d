// Internal layout shared by the host planner and the gfx950 kernels.
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define BBPE_HD __host__ __device__ __forceinline__
#else
#define BBPE_HD inline
#endif

namespace bbpe {

// ---------------------------------------------------------------------------
// Character classes (one code per code point, see gen_unicode_classes.py)
// ---------------------------------------------------------------------------
enum CharClass : uint8_t {
  CC_OTHER = 0, CC_LU = 1, CC_LL = 2, CC_LO = 3, CC_N = 4, CC_WS = 5, CC_M = 6
};

// ---------------------------------------------------------------------------
// Rank hash table: open addressing, linear probing, 16-byte slots.
//   k8   : the first 8 key bytes, little endian, zero padded
//   meta : bits 0-7 key length, bit 8 "self-consistent" (merging the key's
//          own bytes yields exactly this key), bits 9-31 offset of the key in
//          the key blob
//   rank : the id, or -1 for an empty slot
// A parallel array holds key bytes 8..15, so keys of up to 16 bytes compare
// without reading the blob.
// ---------------------------------------------------------------------------
struct Slot {
  uint64_t k8;
  uint32_t meta;
  int32_t rank;
};
static_assert(sizeof(Slot) == 16, "slot is 16 bytes");

constexpr uint32_t META_SELF = 1u << 8;
constexpr uint32_t META_OFF_SHIFT = 9;
constexpr uint32_t MAX_BLOB = 1u << 23;
constexpr int32_t RANK_NONE = 0x7fffffff;  // "pair not in the table"

// MurmurHash3's 64-bit finaliser (Appleby), applied per 8-byte word.
BBPE_HD uint64_t fmix64(uint64_t x) {
  x ^= x >> 33;
  x *= 0xff51afd7ed558ccdull;
  x ^= x >> 33;
  x *= 0xc4ceb9fe1a85ec53ull;
  x ^= x >> 33;
  return x;
}

// Hash of a key given as little-endian zero-padded 8-byte words.
BBPE_HD uint64_t hash_seed(uint32_t len) { return (uint64_t(len) + 1) * 0x9E3779B97F4A7C15ull; }
BBPE_HD uint64_t hash_step(uint64_t h, uint64_t w) { return fmix64(h ^ w); }

// ---------------------------------------------------------------------------
// Merge table: the rank of the key bytes(A) + bytes(B) for every pair of
// keys (A, B) whose concatenation is a key, i.e. every split of a key into
// two keys.  The parts of a piece are always keys, so every lookup the merge
// loop makes after its first round is a lookup of such a pair, and it is
// answered from the two part ids alone.  16-byte buckets of 2 entries (one
// 16-byte load per probe), about a third of the slots used:
//   bit 63 valid | A << 42 | B << 21 | rank      (ids and ranks < 2^21)
// A key hashes to one bucket; a full bucket continues into the next one.
// ---------------------------------------------------------------------------
constexpr uint32_t MT_ID_BITS = 21;
constexpr uint32_t MT_ID_MASK = (1u << MT_ID_BITS) - 1;
constexpr uint32_t MT_BUCKET = 2;
BBPE_HD uint64_t mt_key(uint32_t a, uint32_t b) { return (uint64_t(a) << MT_ID_BITS) | b; }
BBPE_HD uint32_t mt_bucket(uint64_t key, uint32_t shift) {
  return uint32_t((key * 0x9E3779B97F4A7C15ull) >> shift);
}

// Bit of a 4-byte string (little-endian) in the 4-gram bitmap.
BBPE_HD uint32_t q4_index(uint32_t x) { return (x * 0x9E3779B1u) >> 8; }

// ---------------------------------------------------------------------------
// Device view of the uploaded tables (passed to kernels by value).
// ---------------------------------------------------------------------------
struct DevTables {
  const Slot *slots;
  const uint64_t *ext;      // [slots] key bytes 8..15 of each slot's key, zero padded
  const uint8_t *blob;
  const int32_t *pair;      // [65536] rank of the 2-byte key (a,b) at a*256+b, or RANK_NONE
  const int32_t *atom;      // [256] rank of each single byte
  const uint16_t *uni1;     // [4352]
  const uint8_t *uni2;      // [blocks*256]
  const uint8_t *sp_bytes;  // special strings
  const uint32_t *sp_off;   // [n_sp+1]
  const int32_t *sp_id;     // [n_sp]
  const uint32_t *inner;    // [2048] bit (a*256+b): the byte pair (a,b) occurs inside some key
  const uint64_t *mt;       // merge table, [mt_mask+1] buckets of MT_BUCKET entries
  const uint32_t *k3;       // [2^24 bits] bit (a<<16|b<<8|c): the 3-byte string abc is a key
  const uint64_t *dec;      // [dec_n] per rank: offset in dblob << 8 | length, or 0 (no such rank)
  const uint8_t *dblob;     // bytes of every key and special, for decode
  const uint64_t *dsp;      // [2 n_sp] specials sorted by id: id, then offset << 8 | length
  uint32_t dec_n;           // largest rank + 1
  const uint32_t *q4;       // [2^24 bits] bit q4_index(abcd): abcd may occur inside a key
                            //   (every 4-byte substring of a key sets its bit)
  uint32_t mt_mask;
  uint32_t mt_shift;        // 64 - log2(buckets)
  uint32_t slot_mask;
  uint32_t n_sp;
  uint32_t sp_first[8];     // bitmap of first bytes of specials
  uint32_t sp_nfirst;       // distinct first bytes of specials if at most 4, else 0
  uint32_t sp_firsts;       // ... those bytes, one per byte lane
  int32_t grammar;
  uint32_t max_key_len;
  uint32_t sp_overlap;      // 1: two occurrences of specials can overlap (the special pass
                            //    then runs in k_specials)
};

// Byte offsets of each table inside the uploaded image.
struct ImageLayout {
  uint64_t slots, ext, blob, pair, atom, uni1, uni2, sp_bytes, sp_off, sp_id, inner, mt, k3, q4, dec,
      dblob, dsp, total;
  uint32_t n_slots;
  uint32_t n_mt_buckets;
};

// ---------------------------------------------------------------------------
// Text tiling.  A "word" is 64 consecutive text bytes (one lane); a tile is
// one wave of 64 lanes that owns TILE_WORDS words and sees one extra word on
// each side (lanes 0 and 63) for neighbour context.
// ---------------------------------------------------------------------------
constexpr uint32_t TILE_WORDS = 62;
constexpr uint32_t TILE_BYTES = TILE_WORDS * 64;

// Status block at the start of the workspace.
struct Status {
  unsigned long long err_pos;     // first invalid UTF-8 byte (absolute), or ~0
  unsigned long long n_pieces;
  unsigned long long n_ids;
  unsigned long long n_chars;
  unsigned int err_seg;           // segment of err_pos
  unsigned int pad2;              // nonzero: invalid segment offsets, every kernel exits
  unsigned int n_list[8];         // units to merge per length class (MergeList)
  unsigned int scan_ticket;       // next tile of the id-count scan (k_assemble)
  unsigned int scan_fail;         // nonzero: a scan tile's wait for its predecessors gave up
  unsigned int sp_fix;            // nonzero: k_specials left tiles to k_specials_fix
  unsigned int over_cap;          // nonzero: a call's ids exceeded its capacity (host record only)
  unsigned long long wc_hits;     // units settled from the kept word cache (k_probe)
};

// Merge-unit lists by length class: the short tier (one lane per unit,
// positions in registers sized to the class), the group tier (16, 32 or 64
// lanes per unit) and the long tier.
enum MergeList : uint32_t {
  ML_4 = 0,    // 2-4 bytes
  ML_8,        // 5-8
  ML_16,       // 9-16
  ML_32,       // 17-32
  ML_G128,     // 33-128
  ML_G256,     // 129-256
  ML_G512,     // 257-512
  ML_LONG,     // longer
  ML_COUNT
};
// shortest unit of each class (list capacities are text bytes / this)
constexpr uint32_t ML_MIN_LEN[ML_COUNT] = {2, 5, 9, 17, 33, 129, 257, 513};

}  // namespace bbpe
