/*
 * lazy_attn.h -- C ABI of liblazyattn.so: paged attention over a
 * position-agnostic KV cache with the positional encoding deferred into the
 * attention kernels (MI355X / gfx950).
 *
 * Sources (the LazyAttention pages):
 *   [N]  "LazyAttention: Efficient Retrieval-Augmented Generation with Deferred
 *        Positional Encoding", paper notes, papernotes.org
 *   [G]  "LazyAttention: Efficient Retrieval-Augmented Generation with Deferred
 *        Positional Encoding", technical summary, gist.science
 *   [R]  "illinoisdata/lazy-attention", repository landing page
 *
 * Method in one paragraph.  Every cached document is written once, with RoPE
 * applied at its document-local positions 0..L-1 ([N] "Method: overall
 * framework": each document indexed from local position 0; Example 3.1: a
 * cached document "pretends" to sit at 0..|d|).  A request places documents
 * at arbitrary global offsets; inside the fused attention kernel the offset
 * Delta of a document is applied as ONE relative rotation of the query
 * ([N] "Key designs": single relative rotation, never rotate-back-then-
 * forward; RoPE relativity (R_m q)^T (R_n k) = q^T R_{n-m} k, [N]
 * "Background and motivation", [G] "Equivalenza Matematica").  Question and
 * generated tokens are private and keep ordinary RoPE at global positions.
 *
 * Conventions shared by every call:
 *   - The caller owns all memory.  Pointers documented "device" must point to
 *     device memory of the current HIP device; "host" pointers to host memory.
 *     The library allocates no device memory and keeps no state between calls.
 *   - Device work is enqueued on `stream` (a hipStream_t, NULL = the null
 *     stream); the library never synchronises it.
 *   - Arguments are validated on the host before any launch.  A failed check
 *     returns a negative lazy_status, sets lazy_last_error() and launches
 *     nothing.  Launch failures return LAZY_ERR_HIP.
 *   - No C++ exception crosses this ABI.
 *   - Head mapping (GQA / MQA, [N] "Generality"): query head h reads KV head
 *     h / (num_q_heads / num_kv_heads).
 *
 * Data layouts (dh = head_dim, Hkv = num_kv_heads, Hq = num_q_heads, T = element
 * type given by lazy_geom.dtype):
 *   K cache  T [num_blocks][Hkv][16][dh]   token-major inside a block
 *   V cache  T [num_blocks][Hkv][dh][16]   channel-major inside a block
 *   q, out   T [rows][Hq][dh]
 *   k, v     T [tokens][Hkv][dh]           (kv-write inputs)
 *   cos/sin  float [max_pos][dh]: row p holds cos(p*theta_k) at [k] and
 *            sin(p*theta_k) at [dh/2 + k], k = 0..dh/2-1.
 *
 * Tile words ([N] "Key designs": (block id, offset, mask) bit-packed into one
 * 64-bit register and split by shifts inside the kernel; [G] "Implementazione
 * Tecnica", decoding).  One tile = one 16-slot paged block:
 *   bits 63..40 block id (24 bits) | bits 39..16 offset (24 bits) |
 *   bits 15..0 valid-slot mask (bit s set = slot s holds a token).
 * A request's tile list is its context tiles (cached documents) followed by
 * its private tiles (question / generated tokens).  Offset meaning:
 *   context tile, RoPE kinds : Delta, the document's start position
 *   context tile, ALiBi      : global position of the tile's slot 0
 *   private tile, any kind   : global position of the tile's slot 0
 */
#ifndef LAZY_ATTN_H
#define LAZY_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LAZY_OK = 0,
  LAZY_ERR_ARG = -1,         /* an argument is out of range or inconsistent */
  LAZY_ERR_UNSUPPORTED = -2, /* valid request this build does not implement (e.g. head_dim 96) */
  LAZY_ERR_WORKSPACE = -3,   /* workspace missing or smaller than lazy_attn_workspace_size() */
  LAZY_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} lazy_status;

typedef enum { LAZY_BF16 = 0, LAZY_FP32 = 1 } lazy_dtype;

/* Positional-encoding variant; all three share the same kernels and differ in
 * metadata only ([N] "Generality": interleaved / NTK / YaRN RoPE and ALiBi). */
typedef enum {
  LAZY_ROPE_HALF = 0,        /* channel pairs (k, k + dh/2) */
  LAZY_ROPE_INTERLEAVED = 1, /* channel pairs (2k, 2k + 1) */
  LAZY_ALIBI = 2             /* no rotation; score bias -slope_h * (m - n) */
} lazy_pos_kind;

/* Flags in lazy_pos_desc.flags. */
#define LAZY_FLAG_PREROTATED 1u /* control build: context K already at global positions, no deferral */
/* Prefill: the tile lists come from lazy_build_tiles_paired (no tile pair
 * spans two documents, or a document and the private tokens), so the query
 * is rotated once per document (by -Delta, [N] "Key designs": the single
 * relative rotation, here on the query side as the decode applies it)
 * instead of each K tile pair in LDS.  A list without that property gives
 * wrong attention for the pairs that span a boundary; without the flag the
 * prefill rotates K and takes any list. */
#define LAZY_FLAG_DOC_PAIRS 2u

#define LAZY_BLOCK_SIZE 16
#define LAZY_MAX_BLOCK_ID ((1 << 24) - 1)
#define LAZY_MAX_OFFSET ((1 << 24) - 1)

typedef struct {
  int32_t num_q_heads;  /* Hq >= 1, multiple of num_kv_heads, Hq / Hkv <= 128 */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;     /* 64 or 128 */
  int32_t block_size;   /* must be LAZY_BLOCK_SIZE */
  int32_t dtype;        /* lazy_dtype of caches, q, k, v and out */
} lazy_geom;

typedef struct {
  int32_t kind;          /* lazy_pos_kind */
  uint32_t flags;        /* LAZY_FLAG_* */
  int32_t max_pos;       /* rows of cos_sin: every rotation position must be < max_pos (unused when
                            cos_sin is NULL: the in-kernel sincos takes any position < 2^24) */
  float softmax_scale;   /* logit multiplier, e.g. 1/sqrt(dh) (x YaRN temperature gain) */
  const float* cos_sin;  /* device [max_pos][dh]; NULL selects on-the-fly sincos from inv_freq */
  const double* inv_freq;    /* device [dh/2] theta_k; used only when cos_sin == NULL */
  const float* alibi_slopes; /* device [num_q_heads]; required for ALiBi */
} lazy_pos_desc;

/* ---------------------------------------------------------------- host helpers */

/* RoPE frequencies theta_k, k = 0..dh/2-1, in fp64 (host).  yarn_factor <= 1
 * gives textbook theta_k = base^(-2k/dh); yarn_factor > 1 applies YaRN (Peng
 * et al.): r_k = orig_ctx*theta_k/(2 pi), gamma = clamp((r_k - beta_slow) /
 * (beta_fast - beta_slow), 0, 1), theta_k' = (1-gamma) theta_k/s + gamma theta_k.
 * *logit_gain (may be NULL) receives the YaRN temperature gain (0.1 ln s + 1)^2
 * (1 without YaRN) to fold into softmax_scale; it never enters the rotation table.
 * [N] "Generality": scaled RoPE changes metadata only.  Host memory; pure. */
lazy_status lazy_rope_freqs(int32_t head_dim, double base, double yarn_factor, int32_t yarn_orig_ctx,
                            double beta_fast, double beta_slow, double* inv_freq_out, double* logit_gain);

/* Softmax logit multiplier ([N] "Generality": scaled RoPE is metadata): 1/sqrt(head_dim), times the
 * YaRN temperature gain (0.1 ln s + 1)^2 when yarn_factor s > 1 (ALiBi and plain RoPE pass s <= 1).
 * The value callers put in lazy_pos_desc.softmax_scale.  Host; pure. */
lazy_status lazy_softmax_scale(int32_t head_dim, double yarn_factor, float* scale_out);

/* cos/sin table [max_pos][dh] (layout above) from fp64 angles p*theta_k rounded
 * once to fp32 ([N] "Key designs": coefficients from a table, one D-long row
 * per document).  Host memory (caller copies it to the device); pure. */
lazy_status lazy_rope_table(int32_t head_dim, const double* inv_freq, int32_t max_pos, float* table_out);

/* ALiBi slopes 2^(-8 (h+1) / H), h = 0..H-1, as fp32 (host; pure). */
lazy_status lazy_alibi_slopes(int32_t num_heads, float* slopes_out);

/* Pack n tile words (host).  block_ids in [0, 2^24), offsets in [0, 2^24),
 * masks in [1, 0xFFFF]; any value outside its field -> LAZY_ERR_ARG and the
 * index in lazy_last_error().  Pure; out_words[n] caller-allocated. */
lazy_status lazy_pack_tiles(const int64_t* block_ids, const int64_t* offsets, const uint32_t* masks,
                            int64_t n, uint64_t* out_words);

/* Inverse of lazy_pack_tiles on the host (any outputs may be NULL). */
lazy_status lazy_unpack_tiles(const uint64_t* words, int64_t n, int64_t* block_ids, int64_t* offsets,
                              uint32_t* masks);

/* Build every request's tile list from its segments (host).
 *
 * Request r owns segments seg_start[r] .. seg_start[r+1]-1 (seg_start has
 * num_reqs+1 entries, non-decreasing, seg_start[0] = 0).  Segment s holds
 * seg_len[s] >= 0 tokens stored from slot 0 of blocks[seg_block_start[s]]
 * onwards (one block per 16 tokens; seg_block_start has num_segs+1 entries);
 * its first token sits at global position seg_pos0[s].  seg_is_ctx[s] = 1
 * marks a cached document written at local positions (a context segment);
 * 0 marks private tokens written at global positions.  Context segments
 * must precede private ones within a request; among themselves they may come
 * in any order (every tile carries its own offset, and the attention result
 * does not depend on key order beyond rounding).  Listing a batch's shared
 * documents in one common order, most shared first, lets the decode read a
 * shared document for all its requests at about the same time, so that the
 * reads after the first come from L2.
 *
 * Outputs (host, caller-allocated): tiles_out[tiles_cap] words,
 * tile_start[num_reqs+1] (tile range of request r), ctx_tiles[num_reqs]
 * (number of leading context tiles of r).  Block ids must be < num_blocks.
 * max_pos > 0 (the rows of the cos/sin table the attention calls will use)
 * requires every rotary context tile's offset Delta to be < max_pos, since
 * the kernels read row Delta; pass 0 with the in-kernel sincos path or for
 * ALiBi.  A segment of length 0 emits no tile.  Returns LAZY_ERR_ARG if
 * tiles_cap is too small or any field is out of range.  Pure. */
lazy_status lazy_build_tiles(int32_t kind, int32_t num_reqs, const int32_t* seg_start, const int32_t* seg_len,
                             const int64_t* seg_pos0, const uint8_t* seg_is_ctx, const int32_t* seg_block_start,
                             const int32_t* blocks, int64_t num_blocks, int32_t max_pos, uint64_t* tiles_out,
                             int64_t tiles_cap, int32_t* tile_start, int32_t* ctx_tiles);

/* As lazy_build_tiles, with every context segment of an odd tile count
 * closed by one empty tile (block 0, mask 0, the segment's offset), so that
 * each tile pair (2i, 2i+1) of a request lies within one document or within
 * the private tokens: the layout the prefill's per-document query rotation
 * (LAZY_FLAG_DOC_PAIRS) reads.  tiles_cap must allow one extra tile per
 * context segment; ctx_tiles counts the empty tiles. */
lazy_status lazy_build_tiles_paired(int32_t kind, int32_t num_reqs, const int32_t* seg_start,
                                    const int32_t* seg_len, const int64_t* seg_pos0, const uint8_t* seg_is_ctx,
                                    const int32_t* seg_block_start, const int32_t* blocks, int64_t num_blocks,
                                    int32_t max_pos, uint64_t* tiles_out, int64_t tiles_cap, int32_t* tile_start,
                                    int32_t* ctx_tiles);

/* ------------------------------------------------------------- device calls */

/* KV write (the cache-write path, [N] "Method: overall framework"; [G]
 * "Concetto Core").  For each token t < num_tokens:
 *   K cache slot slot_mapping[t] <- R_{positions[t]} k[t]   (RoPE kinds)
 *                                 <- k[t]                   (ALiBi)
 *   V cache slot slot_mapping[t] <- v[t]
 *   q_inout[t]                   <- R_{positions[t]} q[t]   (RoPE kinds, if q_inout != NULL)
 * A document is written with positions 0..L-1 (position-agnostic copy); a
 * question / generated token with its global position.  Slot s addresses
 * block s / 16, slot s % 16.  Device arrays: k, v [T][Hkv][dh]; q_inout
 * [T][Hq][dh] (nullable, updated in place); positions int32 [T];
 * slot_mapping int64 [T].  A token whose slot is negative is not written to
 * the cache (its q is still rotated).  Positions and slots are device data
 * the host cannot see, so callers must validate them before the call
 * (position in [0, max_pos) with a table, [0, 2^24) without; slot <
 * num_blocks*16).  The kernel never reads or writes outside its buffers: a
 * slot >= num_blocks*16 is not written, and a RoPE position that is
 * negative or outside the table turns that token's cache row (and its q
 * row) into NaN, so an invalid position can only show up as NaN outputs,
 * never as silently unrotated keys.
 * Rotation math is fp32; stored values are rounded once to T. */
lazy_status lazy_kv_write(const lazy_geom* geom, const lazy_pos_desc* pos, void* k_cache, void* v_cache,
                          int64_t num_blocks, const void* k, const void* v, void* q_inout,
                          const int32_t* positions, const int64_t* slot_mapping, int32_t num_tokens,
                          void* stream);

/* Bytes of device workspace lazy_attn_prefill / lazy_attn_decode need for
 * these sizes (0 if no workspace is needed).  is_prefill = 0: decode, one
 * query token per request (max_q_len ignored).  max_tiles and total_tiles
 * must be the values later passed to the attention call. */
size_t lazy_attn_workspace_size(const lazy_geom* geom, int32_t num_reqs, int32_t max_q_len, int32_t max_tiles,
                                int64_t total_tiles, int32_t is_prefill);

/* Prefill over cached documents + private suffix ([N] "Key designs":
 * prefill kernel, compute-bound; [G] "Implementazione Tecnica" item 1).
 *
 * Request r has query rows q_start[r] .. q_start[r+1]-1 (q_start: device int32
 * [num_reqs+1]); row i sits at global position q_pos0[r] + (i - q_start[r])
 * (q_pos0: device int32 [num_reqs]) and is already rotated at that position
 * (lazy_kv_write with q_inout).  Its keys are the tiles
 * tiles[tile_start[r] .. tile_start[r+1]-1] (device uint64 / int32 [R+1]) of
 * which the first ctx_tiles[r] (device int32 [R]) are context tiles, fully
 * visible; a private key at global position n is visible to the row at m iff
 * n <= m.  Output out[q rows][Hq][dh] (device, T) = softmax(scale q k'^T +
 * bias) V, k' = the key at its global position (RoPE: rotation by the
 * tile's Delta inside the kernel).  With LAZY_FLAG_DOC_PAIRS in pos->flags
 * (tile lists from lazy_build_tiles_paired) the bf16 kernel applies that
 * rotation to the query instead, once per document (q rotated by -Delta,
 * the same result); without it, to each K tile pair.
 * Host sizing hints: max_q_len >= every request's query count (required);
 * max_tiles ~ the largest tile count and total_tiles ~ tile_start[num_reqs]
 * (0 = unknown) size the split-K plan: each request gets one split per
 * chunk of tiles, so long and short requests finish together.  Wrong tile
 * hints cost speed, never correctness.
 * workspace (device) of ws_bytes >= lazy_attn_workspace_size(..., 1). */
lazy_status lazy_attn_prefill(const lazy_geom* geom, const lazy_pos_desc* pos, const void* k_cache,
                              const void* v_cache, int64_t num_blocks, const uint64_t* tiles,
                              const int32_t* tile_start, const int32_t* ctx_tiles, const void* q,
                              const int32_t* q_start, const int32_t* q_pos0, int32_t num_reqs, int32_t max_q_len,
                              int32_t max_tiles, int64_t total_tiles, void* out, void* workspace, size_t ws_bytes,
                              void* stream);

/* Decode: one new query token per request ([N] "Key designs": decode kernel,
 * bandwidth-bound, M = 1; the query is re-rotated only when the tile's
 * document offset changes; [G] "Implementazione Tecnica" item 2).
 * q: device T [num_reqs][Hq][dh], already rotated at its global position
 * q_pos[r] (device int32 [num_reqs]; read for ALiBi only).  Every valid slot
 * of every tile of the request is visible.  out: device T [num_reqs][Hq][dh].
 * Split-K over tiles with a log-sum-exp combine, planned from the max_tiles /
 * total_tiles hints as for prefill.  workspace as for prefill (is_prefill = 0). */
lazy_status lazy_attn_decode(const lazy_geom* geom, const lazy_pos_desc* pos, const void* k_cache,
                             const void* v_cache, int64_t num_blocks, const uint64_t* tiles,
                             const int32_t* tile_start, const int32_t* ctx_tiles, const void* q,
                             const int32_t* q_pos, int32_t num_reqs, int32_t max_tiles, int64_t total_tiles,
                             void* out, void* workspace, size_t ws_bytes, void* stream);

/* Plan of a document-major decode (host; pure).  Input: the batch's segments
 * as for lazy_build_tiles.  A cached document read by >= min_readers (>= 1)
 * context segments of the batch (one physical copy: same blocks wherever it
 * is read) is "shared": it gets one tile list at its local positions (tile
 * offset = local position of slot 0), and each of its reads a 64-bit read
 * word: request [63:48] | slot [47:32] | Delta [31:0] (slot = index of the
 * read among its request's shared reads; Delta = the document's start in
 * that request, < max_pos when max_pos > 0 for RoPE kinds).  Every request
 * keeps a tile list of its unshared documents and private tokens (same
 * layout as lazy_build_tiles).  With min_readers 1 no document is unshared,
 * and each request's private tokens become one more item of the pass as
 * well: a one-read item whose tiles carry global offsets, read at Delta 0
 * (query and keys both at global positions; no causal mask is needed in
 * decode); the request's own tile list is then empty (remaining tiles 0).
 * Work items: (document, first 16-row block,
 * chunk, tiles per chunk) covering reads x (num_q_heads / num_kv_heads) rows
 * per document, row_blocks x 16 rows each (row_blocks: 8 for bf16, one
 * workgroup of the LDS-staged pass; for fp32 one wave, 2 at dh 128, 4 at
 * dh 64), and the document's tiles in chunks (one per document unless the
 * pass would hold fewer than F work items, F = 256 for bf16 and 1024 for
 * fp32; then up to ceil(2 F / items) even chunks of >= 32 tiles); a read
 * takes one partial slot per chunk of its document, from its slot field on.
 * Outputs (caller-allocated): tiles_out[tiles_cap], tile_start[R+1],
 * ctx_tiles[R]; doc_tiles_out[doc_tiles_cap]; doc_tile_start, read_start
 * [docs_cap+1]; reads_out[reads_cap]; req_reads[R] (shared-read slots per
 * request); work_out[4*work_cap]; counts_out[8] = {documents, reads, work
 * items, max reads of one request, remaining tiles, max remaining tiles of
 * one request, document tiles, row_blocks}.  LAZY_ERR_ARG on a capacity too
 * small or a field out of range. */
lazy_status lazy_build_shared_plan(const lazy_geom* geom, int32_t kind, int32_t num_reqs, const int32_t* seg_start,
                                   const int32_t* seg_len, const int64_t* seg_pos0, const uint8_t* seg_is_ctx,
                                   const int32_t* seg_block_start, const int32_t* blocks, int64_t num_blocks,
                                   int32_t max_pos, int32_t min_readers, uint64_t* tiles_out, int64_t tiles_cap,
                                   int32_t* tile_start, int32_t* ctx_tiles, uint64_t* doc_tiles_out,
                                   int64_t doc_tiles_cap, int32_t* doc_tile_start, int32_t* read_start,
                                   int32_t docs_cap, uint64_t* reads_out, int64_t reads_cap, int32_t* req_reads,
                                   int32_t* work_out, int64_t work_cap, int64_t* counts_out);

/* Bytes of workspace lazy_attn_decode_shared needs (split partials of the
 * requests' own tiles plus one partial slot per shared read). */
size_t lazy_attn_decode_shared_workspace_size(const lazy_geom* geom, int32_t num_reqs, int32_t max_tiles,
                                              int64_t total_tiles, int32_t max_req_reads);

/* Document-major decode ([N] "Key designs": decode rotates the query by the
 * document offset, once per document; [R] README: one position-agnostic copy
 * per document serves every request).  Same result as lazy_attn_decode over
 * each request's full tile list, computed in two passes: (1) each request's
 * own tiles (tiles / tile_start / ctx_tiles of the plan: unshared documents
 * and private tokens), split-K as in lazy_attn_decode, not launched when the
 * plan leaves none (total_tiles 0, as at min_readers 1); (2) every shared
 * document once per KV head for all its reads together: the query of each
 * read is rotated once by -Delta of that read (RoPE; ALiBi measures the
 * key's distance from q_pos - Delta) against the document's keys at their
 * local positions.  A log-sum-exp combine merges each request's partials.
 * Device arrays come from lazy_build_shared_plan (row_blocks =
 * counts_out[7]); q, q_pos, out, cache layouts as for lazy_attn_decode.
 * Needs position-agnostic documents (LAZY_FLAG_PREROTATED is refused).
 * workspace: device, >= lazy_attn_decode_shared_workspace_size(). */
lazy_status lazy_attn_decode_shared(const lazy_geom* geom, const lazy_pos_desc* pos, const void* k_cache,
                                    const void* v_cache, int64_t num_blocks, const uint64_t* tiles,
                                    const int32_t* tile_start, const int32_t* ctx_tiles, int32_t max_tiles,
                                    int64_t total_tiles, const uint64_t* doc_tiles, const int32_t* doc_tile_start,
                                    const int32_t* read_start, const uint64_t* reads, const int32_t* req_reads,
                                    const int32_t* work, int32_t num_docs, int32_t num_work, int32_t max_req_reads,
                                    int32_t row_blocks, const void* q, const int32_t* q_pos, int32_t num_reqs,
                                    void* out, void* workspace, size_t ws_bytes, void* stream);

/* Decode that allocates nothing, for callers that cannot allocate device
 * memory at call time (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, semantics and kernels
 * as lazy_attn_decode, without the workspace: the split-K partials go to a
 * static device array of LAZY_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds for the life of the process (its address is looked
 * up on the first call on each device).  When a batch's plan would need
 * more, it runs with fewer, longer splits that fit; a batch whose query
 * rows (num_reqs x num_q_heads) cannot fit even two splits' partials is
 * refused with LAZY_ERR_WORKSPACE.  The scratch keeps the last call's
 * contents and every call on a device shares it: calls that overlap on one
 * GPU (different streams, different threads) race and must be serialised
 * by the caller.  No hipMalloc, hipFree or allocating library routine is
 * called. */
#define LAZY_NOALLOC_SCRATCH_BYTES (64u << 20)
lazy_status lazy_attn_decode_noalloc(const lazy_geom* geom, const lazy_pos_desc* pos, const void* k_cache,
                                     const void* v_cache, int64_t num_blocks, const uint64_t* tiles,
                                     const int32_t* tile_start, const int32_t* ctx_tiles, const void* q,
                                     const int32_t* q_pos, int32_t num_reqs, int32_t max_tiles, int64_t total_tiles,
                                     void* out, void* stream);

/* Test hook: run the attention kernels' own device-side word unpack on n
 * device words; write device int32 block[n], offset[n], mask[n]. */
lazy_status lazy_debug_unpack(const uint64_t* words, int64_t n, int32_t* block, int32_t* offset, int32_t* mask,
                              void* stream);

/* Message describing the last failure on the calling thread ("" if none). */
const char* lazy_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LAZY_ATTN_H */
