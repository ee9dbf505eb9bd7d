/* bbpe.h -- byte-level BPE encoder for AMD MI355X (gfx950), C ABI.
 *
 * The encode path of a tiktoken-style byte-level BPE tokenizer, run as HIP
 * kernels on one GPU:
 *
 *   * a mergeable-ranks table maps byte strings to ids; the rank is the id and
 *     all 256 single bytes are present, so encoding always terminates
 *     (tiktoken deep-dive page, "An encoding is three objects" and "The byte
 *     floor");
 *   * text arrives as ordered (text, allow_special) segments handled in one
 *     native call; with tiktoken-safe chunking each segment is cut into pieces
 *     of at most 400,000 characters, whose whitespace / non-whitespace runs
 *     are cut at 25,000 characters, and every chunk is encoded as its own
 *     text (Baseten page, "Why Kimi K3 tokenization is non-trivial" and "One
 *     native call for the whole serving path");
 *   * specials are matched by an exact-string pass outside BPE, only in
 *     segments whose allow_special flag is set; elsewhere a literal special
 *     string is ordinary text (tiktoken deep-dive page, "Special tokens");
 *   * each span is cut by a fixed split grammar whose cuts merges never
 *     cross (tiktoken deep-dive page, "The split pattern"; the o200k-style
 *     variant from "r50k, cl100k, o200k");
 *   * each pre-token is merged by repeatedly joining the adjacent pair of
 *     lowest rank, leftmost on ties (tiktoken deep-dive page, "Inside
 *     encode").
 *
 * Conventions.  Every function returns an int status: 0 (BBPE_OK) or a
 * negative BBPE_E_* code.  Functions never throw and never print.  "Host"
 * pointers are ordinary CPU memory; "device" pointers are HIP device memory
 * on the current device.  The caller owns every buffer it passes; the
 * library owns only the opaque tokenizer handle and its host copy of the
 * table.  Device buffers are normally PyTorch tensors: PyTorch provides the
 * memory and the stream, the library provides the kernels.
 */
#ifndef BBPE_H
#define BBPE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque handle.  Its tables are immutable once uploaded.  Host threads may
 * share a handle: every call that enqueues device work or reads or writes
 * its per-handle state (the second stream and its fork/join events, the
 * timing records) holds the handle's lock for its whole duration, so such
 * calls on one handle run one after the other.  For concurrent encodes on
 * one GPU, give each thread its own handle. */
typedef struct bbpe_tokenizer bbpe_tokenizer;

enum {
  BBPE_OK = 0,
  BBPE_E_INVALID_ARG = -1, /* null pointer, bad size, misaligned text, bad flag */
  BBPE_E_TABLE = -2,       /* ranks table violates the format (see load_ranks) */
  BBPE_E_SPECIAL = -3,     /* special-token list violates the format */
  BBPE_E_UTF8 = -4,        /* a segment is not valid UTF-8 (see error_detail) */
  BBPE_E_CAPACITY = -5,    /* ids_capacity too small; *n_ids holds the need */
  BBPE_E_BAD_ID = -6,      /* decode met an id that is neither rank nor special */
  BBPE_E_HIP = -7,         /* a HIP runtime call failed */
  BBPE_E_WORKSPACE = -8,   /* workspace missing or smaller than required */
  BBPE_E_STATE = -9,       /* tables not uploaded yet */
  BBPE_E_NOMEM = -10       /* a host allocation failed */
};

/* Split grammars.  CL100K is the pattern printed on the tiktoken deep-dive
 * page ("The split pattern"), with possessive quantifiers.  O200K_STYLE
 * replaces its first two clauses by one letter clause split by Unicode case
 * categories with the contraction appended to the word ("r50k, cl100k,
 * o200k"):  [^\r\n\p{L}\p{N}]?+ (U*+ W++ | U++ W*+) (?i:'[sdmt]|'ll|'ve|'re)?+
 * with U = [\p{Lu}\p{Lt}\p{Lm}\p{Lo}\p{M}] and W = [\p{Ll}\p{Lm}\p{Lo}\p{M}],
 * followed by the cl100k clauses from the digit clause on.  R50K_STYLE is
 * the cl100k pattern with r50k's digit clause " ?\p{N}++" in place of
 * \p{N}{1,3}+: all the digits of a run form one piece, with no cap on its
 * length, and a single space right before the run joins it (the same page
 * and section give only this clause of r50k's pattern). */
enum { BBPE_GRAMMAR_CL100K = 0, BBPE_GRAMMAR_O200K_STYLE = 1, BBPE_GRAMMAR_R50K_STYLE = 2 };

/* encode flags */
enum {
  BBPE_TIKTOKEN_SAFE = 1u << 0,  /* 400k-character windows, 25k-character run cuts */
  BBPE_COUNT_ONLY = 1u << 1,     /* token counts only: d_id_off and *n_ids are written,
                                    d_ids is not (it may be null, ids_capacity 0) */
  BBPE_KEEP_WORD_CACHE = 1u << 2 /* look units up in, and add them to, the handle's
                                    word cache (see bbpe_word_cache_info) */
};

/* Limits of this implementation. */
#define BBPE_MAX_KEY_BYTES 128u      /* longest mergeable key (tiktoken deep-dive, "The byte floor") */
#define BBPE_MAX_SPECIALS 1024u
#define BBPE_MAX_RANK 2097151u       /* largest rank of a key, 2^21 - 1 (the merge
                                        table packs two ids and a rank in 64 bits;
                                        specials may use any id below 2^31) */
#define BBPE_MAX_SPECIAL_BYTES 64u   /* longest special-token string */

/* Build a tokenizer from a ranks table held in host memory.
 *
 *   key_bytes, key_off[n+1]: key i is key_bytes[key_off[i] .. key_off[i+1]);
 *   ranks[n]:                its rank (= token id), 0 <= rank <= BBPE_MAX_RANK;
 *   special_bytes, special_off[ns+1], special_ids[ns]: special tokens;
 *   grammar:                 BBPE_GRAMMAR_*.
 *
 * Rejected with BBPE_E_TABLE: n == 0, an empty key, a key longer than
 * BBPE_MAX_KEY_BYTES, a duplicate key or rank, a rank outside [0, BBPE_MAX_RANK], or a missing
 * single-byte key (all 256 must be present).  Rejected with BBPE_E_SPECIAL:
 * more than BBPE_MAX_SPECIALS specials, an empty special, one longer than
 * BBPE_MAX_SPECIAL_BYTES, one that is not valid UTF-8, a duplicate string or
 * id, an id that is also a rank, or one special that is a prefix of another
 * (so at most one special can start at any byte).  Specials whose occurrences
 * can overlap in a text (a proper suffix of one equal to a proper prefix of
 * another, as "<|a|>" and "|>b", or one inside another not at its start) are
 * accepted: the encoder takes the leftmost occurrence, resumes the search
 * after its end, and never matches across a segment boundary (tiktoken
 * deep-dive page, "Special tokens").
 * On success *out receives the handle and *device_table_bytes the size of the
 * device memory that bbpe_upload_tables needs.  The library copies what it
 * needs; the caller keeps ownership of every input. */
int bbpe_load_ranks(const uint8_t *key_bytes, const uint64_t *key_off, const int32_t *ranks,
                    uint32_t n, const uint8_t *special_bytes, const uint64_t *special_off,
                    const int32_t *special_ids, uint32_t ns, int grammar,
                    bbpe_tokenizer **out, uint64_t *device_table_bytes);

/* Same, reading tiktoken's text format ("base64(bytes) SP rank LF" per line)
 * from a host file.  BBPE_E_TABLE also covers unreadable files and malformed
 * lines. */
int bbpe_load_ranks_tiktoken_file(const char *path, const uint8_t *special_bytes,
                                  const uint64_t *special_off, const int32_t *special_ids,
                                  uint32_t ns, int grammar, bbpe_tokenizer **out,
                                  uint64_t *device_table_bytes);

/* Copy the device image of the tables (hash table, pair table, Unicode class
 * tables, specials) into caller-owned device memory d_table_mem of at least
 * device_table_bytes bytes, 256-byte aligned, on hip_stream (a hipStream_t,
 * may be null for the null stream).  The memory must stay valid and unchanged
 * for as long as the handle encodes.  Returns after the copy has completed. */
int bbpe_upload_tables(bbpe_tokenizer *tok, void *d_table_mem, uint64_t bytes,
                       void *hip_stream);

/* Device workspace needed to encode total_text_bytes bytes in n_seg segments. */
int bbpe_workspace_bytes(const bbpe_tokenizer *tok, uint64_t total_text_bytes, uint32_t n_seg,
                         uint64_t *out_bytes);

/* Encode n_seg segments in one call.
 *
 *   d_text:           device, the concatenated UTF-8 bytes of all segments,
 *                     16-byte aligned; NUL is an ordinary byte;
 *   total_bytes:      host copy of d_seg_off[n_seg] (the text length, below
 *                     2^32 - 64), so that the call needs no early read-back;
 *   d_seg_off[n_seg+1]: device, uint64 byte offsets; segment s is
 *                     d_text[d_seg_off[s] .. d_seg_off[s+1]); d_seg_off[0]
 *                     must be 0, offsets non-decreasing, and
 *                     d_seg_off[n_seg] == total_bytes (checked on the device:
 *                     BBPE_E_INVALID_ARG otherwise);
 *   d_allow_special[n_seg]: device, 1 = match specials in this segment,
 *                     0 = specials are ordinary text;
 *   flags:            BBPE_TIKTOKEN_SAFE, BBPE_COUNT_ONLY, both or 0 (count-only:
 *                     per-segment token counts for token budgets, no ids);
 *   d_workspace:      device scratch of at least bbpe_workspace_bytes(),
 *                     256-byte aligned; its contents are not preserved;
 *   d_ids:            device output, int32, capacity ids_capacity;
 *   d_id_off[n_seg+1]: device output, int64: the ids of segment s are
 *                     d_ids[d_id_off[s] .. d_id_off[s+1]);
 *   *n_ids:           host output, the number of ids written;
 *   hip_stream:       the stream all work is enqueued on.
 *
 * The total number of ids never exceeds the number of text bytes, so a
 * capacity equal to the byte count always suffices.  With a smaller capacity
 * the call returns BBPE_E_CAPACITY, sets *n_ids to the count needed and
 * leaves d_ids unspecified.  Invalid UTF-8 in any segment returns
 * BBPE_E_UTF8; bbpe_error_detail then reports the first offending segment and
 * byte.  The call synchronises the stream once, at its end, to read the
 * status and *n_ids; that is its only host synchronisation.
 *
 * With BBPE_COUNT_ONLY the call writes d_id_off and *n_ids only: the per-
 * segment token counts are d_id_off[s+1] - d_id_off[s] (token budgets: the
 * tiktoken deep-dive page, "Counting tokens for a budget"); d_ids may
 * be null and no capacity error is returned. */
int bbpe_encode_segments(bbpe_tokenizer *tok, const uint8_t *d_text, uint64_t total_bytes,
                         const uint64_t *d_seg_off, const uint8_t *d_allow_special,
                         uint32_t n_seg, uint32_t flags,
                         void *d_workspace, uint64_t workspace_bytes, int32_t *d_ids,
                         uint64_t ids_capacity, int64_t *d_id_off, uint64_t *n_ids,
                         void *hip_stream);

/* bbpe_encode_segments without the wait: the same arguments but n_ids, and
 * the same work, enqueued on hip_stream; returns once it is enqueued, so a
 * serving loop can queue the next batch while this one runs (the Baseten
 * page, "One native call for the whole serving path": every crossing of the
 * native boundary costs, and here each blocking call also costs a host round
 * trip between batches).  The call's id count is d_id_off[n_seg] on the
 * device.  Calls enqueued this way and not yet waited for are outstanding;
 * while any is, every encode or pre-tokenize call on the handle must use the
 * same stream (BBPE_E_INVALID_ARG otherwise), and they run in stream order,
 * so they may share a workspace.  Errors come from bbpe_encode_wait (or from
 * the next synchronous call on the handle, which settles the outstanding
 * ones too).  Arguments checked on the host return their error at once, and
 * nothing is enqueued.  BBPE_E_STATE while per-kernel timing is on. */
int bbpe_encode_segments_async(bbpe_tokenizer *tok, const uint8_t *d_text, uint64_t total_bytes,
                               const uint64_t *d_seg_off, const uint8_t *d_allow_special,
                               uint32_t n_seg, uint32_t flags, void *d_workspace,
                               uint64_t workspace_bytes, int32_t *d_ids, uint64_t ids_capacity,
                               int64_t *d_id_off, void *hip_stream);

/* Waits for every outstanding bbpe_encode_segments_async call of the handle
 * (hip_stream must be theirs: BBPE_E_INVALID_ARG otherwise; BBPE_E_STATE if
 * none is outstanding).  *n_ids (host) receives the last call's id count.
 * The result is the first error any of them met, in this order: bad segment
 * offsets (BBPE_E_INVALID_ARG), a device-side wait of the ordered assembly
 * that gave up (BBPE_E_HIP), invalid UTF-8 (BBPE_E_UTF8, the first such
 * byte met kept for bbpe_error_detail), ids beyond a call's capacity
 * (BBPE_E_CAPACITY), else BBPE_OK. */
int bbpe_encode_wait(bbpe_tokenizer *tok, void *hip_stream, uint64_t *n_ids);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * bbpe_encode_segments without a workspace argument.  Same arguments
 * (d_workspace and workspace_bytes aside), results, errors and
 * synchronisation.  Its workspace is a static device array of
 * BBPE_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held
 * from the library's first use of that GPU until the process ends; the
 * call allocates nothing and creates no stream or event, and runs every
 * kernel on hip_stream (which must belong to the current device).  Texts
 * whose workspace (bbpe_workspace_bytes, some 50 bytes per text byte)
 * exceeds the array -- about a megabyte of text -- return
 * BBPE_E_WORKSPACE.  All calls of this entry point in one process share the
 * array and run one at a time (a lock); calls from other processes use
 * their own copy. */
#define BBPE_NOALLOC_SCRATCH_BYTES (48ull << 20)
int bbpe_encode_segments_noalloc(bbpe_tokenizer *tok, const uint8_t *d_text,
                                 uint64_t total_bytes, const uint64_t *d_seg_off,
                                 const uint8_t *d_allow_special, uint32_t n_seg, uint32_t flags,
                                 int32_t *d_ids, uint64_t ids_capacity, int64_t *d_id_off,
                                 uint64_t *n_ids, void *hip_stream);

/* Pre-tokenization only: the same segment handling, chunking, special pass
 * and split as bbpe_encode_segments, without merging.  Writes the byte offset
 * (into d_text) of every piece in text order to d_starts (device, uint32,
 * capacity starts_cap) and, when d_is_special is not null, 1 for pieces that
 * are special tokens and 0 otherwise (device, uint8).  *n_pieces (host)
 * receives the count; BBPE_E_CAPACITY if it exceeds starts_cap.  Pieces
 * never cross a chunk cut, a special or a segment boundary (tiktoken
 * deep-dive page, "The split pattern": merges never cross a cut).  Same
 * arguments, errors and synchronisation as bbpe_encode_segments
 * (BBPE_COUNT_ONLY is not accepted here: BBPE_E_INVALID_ARG). */
int bbpe_pretokenize_segments(bbpe_tokenizer *tok, const uint8_t *d_text, uint64_t total_bytes,
                              const uint64_t *d_seg_off, const uint8_t *d_allow_special,
                              uint32_t n_seg, uint32_t flags, void *d_workspace,
                              uint64_t workspace_bytes, uint32_t *d_starts, uint64_t starts_cap,
                              uint8_t *d_is_special, uint64_t *n_pieces, void *hip_stream);

/* Decode host ids to bytes (host memory): the concatenation of each token's
 * bytes; specials decode to their strings.  The result is bytes, not text: a
 * token may end inside a UTF-8 character (tiktoken deep-dive page, "Pitfalls
 * that bite in production").  Returns BBPE_E_BAD_ID for an id that is neither
 * a rank nor a special (*out_len = its index), BBPE_E_CAPACITY if cap is too
 * small (*out_len = bytes needed). */
int bbpe_decode(const bbpe_tokenizer *tok, const int32_t *ids, uint64_t n, uint8_t *out,
                uint64_t cap, uint64_t *out_len);

/* Decode on the device.  d_ids[n_ids] (device, int32) -> d_out (device,
 * capacity out_capacity): the concatenation of each token's bytes, specials
 * decoded to their strings (tiktoken deep-dive page, "An encoding is three
 * objects").  When d_tok_off (device, uint64[n_ids]) is not null it receives
 * each token's byte offset in the output, which for the ids of one encode
 * call is the token's byte offset in the text it came from.  *out_len (host)
 * receives the output length; *complete_len (host, may be null) the length of
 * the longest prefix that ends on a complete UTF-8 character, so that a
 * streaming caller can hold back a partial character (a token may end inside
 * one: tiktoken deep-dive page, "Pitfalls that bite in production").  d_workspace: device, at least
 * bbpe_decode_workspace_bytes(), 256-byte aligned.  Returns BBPE_E_BAD_ID for
 * an id that is neither a rank nor a special (*out_len = the index of the
 * first), BBPE_E_CAPACITY when out_capacity is too small (*out_len = bytes
 * needed; d_out is then not written, d_tok_off is).  Enqueues on hip_stream
 * and synchronises it once, at the end.  d_ids must be 4-byte and d_tok_off
 * 8-byte aligned (16-byte alignment of both is faster), n_ids below 2^40:
 * BBPE_E_INVALID_ARG otherwise. */
int bbpe_decode_workspace_bytes(const bbpe_tokenizer *tok, uint64_t n_ids, uint64_t *out_bytes);
int bbpe_decode_device(bbpe_tokenizer *tok, const int32_t *d_ids, uint64_t n_ids,
                       uint8_t *d_out, uint64_t out_capacity, uint64_t *d_tok_off,
                       void *d_workspace, uint64_t workspace_bytes, uint64_t *out_len,
                       uint64_t *complete_len, void *hip_stream);

/* Stateful streaming decode (tiktoken deep-dive page, "Pitfalls that bite
 * in production": a token can end inside a UTF-8 character, so text that is
 * shown as it is generated must hold back a trailing partial character until
 * the tokens that complete it arrive).  A stream decoder keeps, between
 * calls, the bytes of the trailing partial character of everything it has
 * decoded (at most 3).  Each call decodes d_ids[n_ids] (device, int32) on
 * the device and writes to d_out (device, capacity out_capacity) the held
 * bytes followed by the ids' bytes; *out_len (host) receives how many of
 * them are emitted: all of them when final != 0 (the decoder is then empty),
 * else the longest prefix that ends on a complete UTF-8 character, the rest
 * being held for the next call (bytes that cannot start or continue a
 * well-formed character are emitted as they are).  Concatenating the
 * emitted bytes of a sequence of calls, the last one final, gives the decode
 * of all of their ids.  d_out receives up to out_len + 3 bytes.  Workspace,
 * alignment, stream and synchronisation as bbpe_decode_device.  Errors leave
 * the held bytes unchanged: BBPE_E_BAD_ID (*out_len = index of the first bad
 * id in this call), BBPE_E_CAPACITY (*out_len = bytes needed).  A decoder
 * belongs to one caller at a time (calls on one decoder must not overlap);
 * it keeps a pointer to tok, which must outlive it.  bbpe_stream_decoder_reset
 * drops the held bytes. */
typedef struct bbpe_stream_decoder bbpe_stream_decoder;
int bbpe_stream_decoder_create(bbpe_tokenizer *tok, bbpe_stream_decoder **out);
int bbpe_stream_decoder_free(bbpe_stream_decoder *dec);
int bbpe_stream_decoder_reset(bbpe_stream_decoder *dec);
int bbpe_stream_decode_device(bbpe_stream_decoder *dec, const int32_t *d_ids, uint64_t n_ids, int final,
                              uint8_t *d_out, uint64_t out_capacity, void *d_workspace,
                              uint64_t workspace_bytes, uint64_t *out_len, void *hip_stream);

/* Per-token byte offsets without decoding: d_tok_off[i] (device, uint64,
 * n_ids entries, 8-byte aligned) receives the byte offset of token i, that
 * is the total length of the bytes of tokens 0..i-1; for the ids of one
 * encode call it is the token's byte offset in the encoded text: a field of
 * an encoding besides its ids, computed only when asked for (Kimi K3
 * tokenization page, "Where the speed comes from": encodings are
 * materialised when accessed).  *total_bytes (host) receives the length of the whole
 * decode.  Same workspace (bbpe_decode_workspace_bytes), alignment rules,
 * stream and synchronisation as bbpe_decode_device; BBPE_E_BAD_ID with
 * *total_bytes = the index of the first bad id. */
int bbpe_token_offsets_device(bbpe_tokenizer *tok, const int32_t *d_ids, uint64_t n_ids,
                              uint64_t *d_tok_off, void *d_workspace, uint64_t workspace_bytes,
                              uint64_t *total_bytes, void *hip_stream);

/* The word cache kept across calls (tokenizers v1 page, "Key Technical
 * Improvements": a cache of the ids of words already merged).  Units of 2-32
 * bytes that need the merge loop are looked up by their bytes in a device
 * hash table held by the handle; the ones found take their ids from it, and
 * the ones merged are added to it, for the calls that follow.  Only calls of
 * bbpe_encode_segments with BBPE_KEEP_WORD_CACHE use it (the first such call
 * allocates it, BBPE_WORD_CACHE_ENTRIES entries of 128 bytes, on the current
 * device; bbpe_encode_segments_noalloc rejects the flag with
 * BBPE_E_INVALID_ARG).  The cache holds the merge results of this handle's
 * table only, so its answers are exact; it is best-effort in what it holds
 * (a unit whose slots are taken is not added; nothing is evicted).
 * bbpe_word_cache_clear empties it (on hip_stream, synchronised);
 * bbpe_word_cache_info gives its capacity in entries (0 before it is
 * allocated) and how many units the last BBPE_KEEP_WORD_CACHE call took
 * from it. */
#define BBPE_WORD_CACHE_ENTRIES (1u << 18)
int bbpe_word_cache_clear(bbpe_tokenizer *tok, void *hip_stream);
int bbpe_word_cache_info(bbpe_tokenizer *tok, uint64_t *entries, uint64_t *last_hits);

/* Details of the last BBPE_E_UTF8 that bbpe_encode_segments or
 * bbpe_pretokenize_segments returned to the calling thread on this handle:
 * the segment index and the absolute byte offset in d_text of the first
 * invalid sequence (0 and 0 when there was none). */
int bbpe_error_detail(const bbpe_tokenizer *tok, uint32_t *segment, uint64_t *byte_offset);

/* Number of ranks and the largest id (rank or special) of the table. */
int bbpe_table_info(const bbpe_tokenizer *tok, uint32_t *n_ranks, int32_t *max_id,
                    uint32_t *n_specials, int *grammar);

/* Diagnostics: per-kernel device time.  With timing enabled, every later
 * encode or pretokenize call on this handle brackets each kernel launch with
 * a pair of HIP events on the call's stream and, after the call's final
 * synchronisation, adds the elapsed time to that kernel's running total.
 * bbpe_timing_report returns, for kernel index idx (0, 1, ... until it
 * returns BBPE_E_INVALID_ARG), its name (a static string), the total
 * milliseconds and the number of launches since the last reset. */
int bbpe_set_timing(bbpe_tokenizer *tok, int enable);
int bbpe_timing_report(const bbpe_tokenizer *tok, uint32_t idx, const char **name,
                       double *total_ms, uint64_t *launches);
int bbpe_timing_reset(bbpe_tokenizer *tok);

void bbpe_free(bbpe_tokenizer *tok);

/* A static English description of a status code. */
const char *bbpe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* BBPE_H */
