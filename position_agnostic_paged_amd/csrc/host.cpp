// Host-side part of liblazyattn: error text, argument validation, the
// positional-encoding metadata (RoPE / YaRN frequencies, cos/sin table, ALiBi
// slopes) and the tile-word packer / per-request tile builder.  Pure host
// code; nothing here touches the GPU.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <unordered_map>
#include <vector>

#include "lazy_host.hpp"

namespace lazy {

static thread_local std::string g_err;

lazy_status fail(lazy_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

void clear_error() { g_err.clear(); }

lazy_status check_geom(const lazy_geom* g) {
  if (!g) return fail(LAZY_ERR_ARG, "geom is NULL");
  if (g->num_kv_heads < 1 || g->num_q_heads < 1)
    return fail(LAZY_ERR_ARG, "head counts must be >= 1 (Hq=%d, Hkv=%d)", g->num_q_heads, g->num_kv_heads);
  if (g->num_q_heads % g->num_kv_heads != 0)
    return fail(LAZY_ERR_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", g->num_q_heads,
                g->num_kv_heads);
  if (g->num_q_heads / g->num_kv_heads > 128)
    return fail(LAZY_ERR_UNSUPPORTED, "more than 128 query heads per KV head");
  if (g->head_dim != 64 && g->head_dim != 128)
    return fail(LAZY_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", g->head_dim);
  if (g->block_size != LAZY_BLOCK_SIZE)
    return fail(LAZY_ERR_UNSUPPORTED, "block_size must be %d (got %d)", LAZY_BLOCK_SIZE, g->block_size);
  if (g->dtype != LAZY_BF16 && g->dtype != LAZY_FP32) return fail(LAZY_ERR_ARG, "unknown dtype %d", g->dtype);
  return LAZY_OK;
}

lazy_status check_pos(const lazy_geom* g, const lazy_pos_desc* p) {
  if (!p) return fail(LAZY_ERR_ARG, "pos descriptor is NULL");
  if (p->kind != LAZY_ROPE_HALF && p->kind != LAZY_ROPE_INTERLEAVED && p->kind != LAZY_ALIBI)
    return fail(LAZY_ERR_ARG, "unknown positional kind %d", p->kind);
  if (p->flags & ~(LAZY_FLAG_PREROTATED | LAZY_FLAG_DOC_PAIRS))
    return fail(LAZY_ERR_ARG, "unknown flags 0x%x", p->flags);
  if (!(p->softmax_scale > 0.f) || !isfinite(p->softmax_scale))
    return fail(LAZY_ERR_ARG, "softmax_scale must be finite and > 0");
  if (p->kind == LAZY_ALIBI) {
    if (!p->alibi_slopes) return fail(LAZY_ERR_ARG, "ALiBi needs alibi_slopes");
    (void)g;
    return LAZY_OK;
  }
  if (p->cos_sin) {
    if (p->max_pos < 1) return fail(LAZY_ERR_ARG, "max_pos must be >= 1 with a cos/sin table");
  } else if (!p->inv_freq) {
    return fail(LAZY_ERR_ARG, "RoPE needs cos_sin or inv_freq");
  }
  return LAZY_OK;
}

}  // namespace lazy

using namespace lazy;

extern "C" const char* lazy_last_error(void) { return g_err.c_str(); }

extern "C" lazy_status lazy_rope_freqs(int32_t head_dim, double base, double yarn_factor, int32_t yarn_orig_ctx,
                                       double beta_fast, double beta_slow, double* inv_freq_out,
                                       double* logit_gain) {
  clear_error();
  if (head_dim < 2 || head_dim % 2) return fail(LAZY_ERR_ARG, "head_dim must be even and >= 2");
  if (!(base > 1.0)) return fail(LAZY_ERR_ARG, "base must be > 1");
  if (!inv_freq_out) return fail(LAZY_ERR_ARG, "inv_freq_out is NULL");
  const bool yarn = yarn_factor > 1.0;
  if (yarn && (yarn_orig_ctx < 1 || !(beta_fast > beta_slow)))
    return fail(LAZY_ERR_ARG, "YaRN needs orig_ctx >= 1 and beta_fast > beta_slow");
  const int half = head_dim / 2;
  const double two_pi = 6.283185307179586476925286766559;
  for (int k = 0; k < half; ++k) {
    // textbook RoPE frequency base^(-2k/dh)
    const double theta = pow(base, -(double)(2 * k) / (double)head_dim);
    double f = theta;
    if (yarn) {
      // YaRN "NTK-by-parts": r = rotations of this pair over the original
      // context; linear ramp between beta_slow and beta_fast rotations blends
      // interpolation (theta / s) with extrapolation (theta).
      const double r = (double)yarn_orig_ctx * theta / two_pi;
      double gamma = (r - beta_slow) / (beta_fast - beta_slow);
      gamma = gamma < 0.0 ? 0.0 : (gamma > 1.0 ? 1.0 : gamma);
      f = (1.0 - gamma) * theta / yarn_factor + gamma * theta;
    }
    inv_freq_out[k] = f;
  }
  if (logit_gain) {
    const double t = yarn ? 0.1 * log(yarn_factor) + 1.0 : 1.0;
    *logit_gain = t * t;
  }
  return LAZY_OK;
}

extern "C" lazy_status lazy_softmax_scale(int32_t head_dim, double yarn_factor, float* scale_out) {
  clear_error();
  if (head_dim < 1) return fail(LAZY_ERR_ARG, "head_dim must be >= 1");
  if (!scale_out) return fail(LAZY_ERR_ARG, "scale_out is NULL");
  // 1/sqrt(dh) on the logits; YaRN adds its temperature gain (0.1 ln s + 1)^2
  const double t = yarn_factor > 1.0 ? 0.1 * log(yarn_factor) + 1.0 : 1.0;
  *scale_out = (float)(t * t / sqrt((double)head_dim));
  return LAZY_OK;
}

extern "C" lazy_status lazy_rope_table(int32_t head_dim, const double* inv_freq, int32_t max_pos, float* table_out) {
  clear_error();
  if (head_dim < 2 || head_dim % 2) return fail(LAZY_ERR_ARG, "head_dim must be even and >= 2");
  if (max_pos < 1) return fail(LAZY_ERR_ARG, "max_pos must be >= 1");
  if (!inv_freq || !table_out) return fail(LAZY_ERR_ARG, "NULL pointer");
  const int half = head_dim / 2;
  for (int64_t p = 0; p < max_pos; ++p) {
    float* row = table_out + p * head_dim;
    for (int k = 0; k < half; ++k) {
      const double phi = (double)p * inv_freq[k];
      row[k] = (float)cos(phi);
      row[half + k] = (float)sin(phi);
    }
  }
  return LAZY_OK;
}

extern "C" lazy_status lazy_alibi_slopes(int32_t num_heads, float* slopes_out) {
  clear_error();
  if (num_heads < 1 || !slopes_out) return fail(LAZY_ERR_ARG, "num_heads must be >= 1 and slopes_out non-NULL");
  for (int h = 0; h < num_heads; ++h) slopes_out[h] = (float)exp2(-8.0 * (double)(h + 1) / (double)num_heads);
  return LAZY_OK;
}

extern "C" lazy_status lazy_pack_tiles(const int64_t* block_ids, const int64_t* offsets, const uint32_t* masks,
                                       int64_t n, uint64_t* out_words) {
  clear_error();
  if (n < 0) return fail(LAZY_ERR_ARG, "n must be >= 0");
  if (n > 0 && (!block_ids || !offsets || !masks || !out_words)) return fail(LAZY_ERR_ARG, "NULL pointer");
  for (int64_t i = 0; i < n; ++i) {
    if (block_ids[i] < 0 || block_ids[i] > LAZY_MAX_BLOCK_ID)
      return fail(LAZY_ERR_ARG, "tile %lld: block id %lld outside [0, 2^24)", (long long)i, (long long)block_ids[i]);
    if (offsets[i] < 0 || offsets[i] > LAZY_MAX_OFFSET)
      return fail(LAZY_ERR_ARG, "tile %lld: offset %lld outside [0, 2^24)", (long long)i, (long long)offsets[i]);
    if (masks[i] == 0 || masks[i] > 0xFFFFu)
      return fail(LAZY_ERR_ARG, "tile %lld: mask 0x%x outside [1, 0xFFFF]", (long long)i, masks[i]);
    out_words[i] = ((uint64_t)block_ids[i] << 40) | ((uint64_t)offsets[i] << 16) | (uint64_t)masks[i];
  }
  return LAZY_OK;
}

extern "C" lazy_status lazy_unpack_tiles(const uint64_t* words, int64_t n, int64_t* block_ids, int64_t* offsets,
                                         uint32_t* masks) {
  clear_error();
  if (n < 0) return fail(LAZY_ERR_ARG, "n must be >= 0");
  if (n > 0 && !words) return fail(LAZY_ERR_ARG, "NULL words");
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t w = words[i];
    if (block_ids) block_ids[i] = (int64_t)(w >> 40);
    if (offsets) offsets[i] = (int64_t)((w >> 16) & 0xFFFFFFull);
    if (masks) masks[i] = (uint32_t)(w & 0xFFFFull);
  }
  return LAZY_OK;
}

namespace lazy {
namespace {

// Checks shared by the tile builders: kind, counts, array presence.
lazy_status check_segments(int32_t kind, int32_t num_reqs, const int32_t* seg_start, const int32_t* seg_len,
                           const int64_t* seg_pos0, const uint8_t* seg_is_ctx, const int32_t* seg_block_start,
                           const int32_t* blocks, int64_t num_blocks) {
  if (kind != LAZY_ROPE_HALF && kind != LAZY_ROPE_INTERLEAVED && kind != LAZY_ALIBI)
    return fail(LAZY_ERR_ARG, "unknown positional kind %d", kind);
  if (num_reqs < 0) return fail(LAZY_ERR_ARG, "num_reqs must be >= 0");
  if (!seg_start) return fail(LAZY_ERR_ARG, "NULL pointer");
  if (seg_start[0] != 0) return fail(LAZY_ERR_ARG, "seg_start[0] must be 0");
  const int32_t nseg = seg_start[num_reqs];
  if (nseg > 0 && (!seg_len || !seg_pos0 || !seg_is_ctx || !seg_block_start || !blocks))
    return fail(LAZY_ERR_ARG, "NULL segment array");
  if (num_blocks < 1 || num_blocks > (int64_t)LAZY_MAX_BLOCK_ID + 1)
    return fail(LAZY_ERR_ARG, "num_blocks must be in [1, 2^24]");
  for (int r = 0; r < num_reqs; ++r)
    if (seg_start[r + 1] < seg_start[r]) return fail(LAZY_ERR_ARG, "seg_start decreases at request %d", r);
  return LAZY_OK;
}

// Emits the tile words of segment s (offset rule of the header) into
// out[nt...]; validates its fields.
lazy_status emit_segment(int32_t kind, int s, const int32_t* seg_len, const int64_t* seg_pos0,
                         const uint8_t* seg_is_ctx, const int32_t* seg_block_start, const int32_t* blocks,
                         int64_t num_blocks, int32_t max_pos, uint64_t* out, int64_t cap, int64_t& nt) {
  const int32_t L = seg_len[s];
  const int64_t p0 = seg_pos0[s];
  const bool ctx = seg_is_ctx[s] != 0;
  if (L < 0) return fail(LAZY_ERR_ARG, "segment %d: negative length", s);
  if (p0 < 0) return fail(LAZY_ERR_ARG, "segment %d: negative position", s);
  const int32_t nblk = (L + LAZY_BLOCK_SIZE - 1) / LAZY_BLOCK_SIZE;
  if (seg_block_start[s + 1] - seg_block_start[s] < nblk)
    return fail(LAZY_ERR_ARG, "segment %d: %d blocks for %d tokens", s, seg_block_start[s + 1] - seg_block_start[s], L);
  for (int32_t b = 0; b < nblk; ++b) {
    const int64_t blk = blocks[seg_block_start[s] + b];
    const int32_t valid = (L - LAZY_BLOCK_SIZE * b) < LAZY_BLOCK_SIZE ? (L - LAZY_BLOCK_SIZE * b) : LAZY_BLOCK_SIZE;
    const uint32_t mask = (uint32_t)((1u << valid) - 1u);
    // rotary context tile: the document's start (the rotation amount);
    // otherwise the global position of the tile's first slot
    const int64_t off = (ctx && kind != LAZY_ALIBI) ? p0 : p0 + (int64_t)LAZY_BLOCK_SIZE * b;
    if (blk < 0 || blk >= num_blocks)
      return fail(LAZY_ERR_ARG, "segment %d block %d: id %lld outside the pool", s, b, (long long)blk);
    if (off > LAZY_MAX_OFFSET) return fail(LAZY_ERR_ARG, "segment %d: offset %lld exceeds 2^24-1", s, (long long)off);
    // the kernels read cos/sin row Delta of every rotary context tile
    if (max_pos > 0 && ctx && kind != LAZY_ALIBI && off >= max_pos)
      return fail(LAZY_ERR_ARG, "segment %d: document offset %lld outside the cos/sin table (max_pos %d)", s,
                  (long long)off, max_pos);
    if (nt >= cap) return fail(LAZY_ERR_ARG, "tile capacity %lld too small", (long long)cap);
    out[nt++] = ((uint64_t)blk << 40) | ((uint64_t)off << 16) | (uint64_t)mask;
  }
  return LAZY_OK;
}

}  // namespace
}  // namespace lazy

namespace {

lazy_status build_tiles(int32_t kind, int32_t num_reqs, const int32_t* seg_start, const int32_t* seg_len,
                        const int64_t* seg_pos0, const uint8_t* seg_is_ctx, const int32_t* seg_block_start,
                        const int32_t* blocks, int64_t num_blocks, int32_t max_pos, bool align_pairs,
                        uint64_t* tiles_out, int64_t tiles_cap, int32_t* tile_start, int32_t* ctx_tiles) {
  clear_error();
  lazy_status st = check_segments(kind, num_reqs, seg_start, seg_len, seg_pos0, seg_is_ctx, seg_block_start, blocks,
                                  num_blocks);
  if (st != LAZY_OK) return st;
  if (!tile_start || !ctx_tiles) return fail(LAZY_ERR_ARG, "NULL pointer");
  int64_t nt = 0;
  for (int r = 0; r < num_reqs; ++r) {
    if (nt > INT32_MAX) return fail(LAZY_ERR_ARG, "too many tiles");
    tile_start[r] = (int32_t)nt;
    bool seen_private = false;
    int64_t nctx = 0;
    for (int s = seg_start[r]; s < seg_start[r + 1]; ++s) {
      const bool ctx = seg_is_ctx[s] != 0;
      if (ctx && seen_private) return fail(LAZY_ERR_ARG, "request %d: context segment %d after a private one", r, s);
      if (!ctx) seen_private = true;
      const int64_t before = nt;
      st = emit_segment(kind, s, seg_len, seg_pos0, seg_is_ctx, seg_block_start, blocks, num_blocks, max_pos,
                        tiles_out, tiles_cap, nt);
      if (st != LAZY_OK) return st;
      if (ctx && align_pairs && ((nt - before) & 1)) {
        // one empty tile (mask 0, block 0, the segment's offset) closes the
        // document's last pair
        if (nt >= tiles_cap) return fail(LAZY_ERR_ARG, "tile capacity %lld too small", (long long)tiles_cap);
        const int64_t nblk = nt - before;
        const int64_t off = kind != LAZY_ALIBI ? seg_pos0[s] : seg_pos0[s] + (int64_t)LAZY_BLOCK_SIZE * nblk;
        if (off > LAZY_MAX_OFFSET) return fail(LAZY_ERR_ARG, "segment %d: offset %lld exceeds 2^24-1", s, (long long)off);
        tiles_out[nt++] = (uint64_t)off << 16;
      }
      if (ctx) nctx += nt - before;
    }
    ctx_tiles[r] = (int32_t)nctx;
  }
  if (nt > INT32_MAX) return fail(LAZY_ERR_ARG, "too many tiles");
  tile_start[num_reqs] = (int32_t)nt;
  return LAZY_OK;
}

}  // namespace

extern "C" lazy_status lazy_build_tiles(int32_t kind, int32_t num_reqs, const int32_t* seg_start,
                                        const int32_t* seg_len, const int64_t* seg_pos0, const uint8_t* seg_is_ctx,
                                        const int32_t* seg_block_start, const int32_t* blocks, int64_t num_blocks,
                                        int32_t max_pos, uint64_t* tiles_out, int64_t tiles_cap,
                                        int32_t* tile_start, int32_t* ctx_tiles) {
  return build_tiles(kind, num_reqs, seg_start, seg_len, seg_pos0, seg_is_ctx, seg_block_start, blocks, num_blocks,
                     max_pos, false, tiles_out, tiles_cap, tile_start, ctx_tiles);
}

extern "C" lazy_status lazy_build_tiles_paired(int32_t kind, int32_t num_reqs, const int32_t* seg_start,
                                               const int32_t* seg_len, const int64_t* seg_pos0,
                                               const uint8_t* seg_is_ctx, const int32_t* seg_block_start,
                                               const int32_t* blocks, int64_t num_blocks, int32_t max_pos,
                                               uint64_t* tiles_out, int64_t tiles_cap, int32_t* tile_start,
                                               int32_t* ctx_tiles) {
  return build_tiles(kind, num_reqs, seg_start, seg_len, seg_pos0, seg_is_ctx, seg_block_start, blocks, num_blocks,
                     max_pos, true, tiles_out, tiles_cap, tile_start, ctx_tiles);
}

extern "C" lazy_status lazy_build_shared_plan(
    const lazy_geom* geom, int32_t kind, int32_t num_reqs, const int32_t* seg_start, const int32_t* seg_len,
    const int64_t* seg_pos0, const uint8_t* seg_is_ctx, const int32_t* seg_block_start, const int32_t* blocks,
    int64_t num_blocks, int32_t max_pos, int32_t min_readers, uint64_t* tiles_out, int64_t tiles_cap,
    int32_t* tile_start, int32_t* ctx_tiles, uint64_t* doc_tiles_out, int64_t doc_tiles_cap, int32_t* doc_tile_start,
    int32_t* read_start, int32_t docs_cap, uint64_t* reads_out, int64_t reads_cap, int32_t* req_reads,
    int32_t* work_out, int64_t work_cap, int64_t* counts_out) {
  clear_error();
  lazy_status st = check_geom(geom);
  if (st != LAZY_OK) return st;
  st = check_segments(kind, num_reqs, seg_start, seg_len, seg_pos0, seg_is_ctx, seg_block_start, blocks, num_blocks);
  if (st != LAZY_OK) return st;
  if (min_readers < 1) return fail(LAZY_ERR_ARG, "min_readers must be >= 1 (got %d)", min_readers);
  if (num_reqs > 65536) return fail(LAZY_ERR_UNSUPPORTED, "more than 65536 requests");
  if (!tile_start || !ctx_tiles || !doc_tile_start || !read_start || !req_reads || !counts_out)
    return fail(LAZY_ERR_ARG, "NULL output array");
  const int32_t nseg = seg_start[num_reqs];

  // 1. readers of every cached document (one physical copy: same first block
  //    and length wherever it is read)
  std::unordered_map<uint64_t, int32_t> readers;
  auto key_of = [&](int s) -> uint64_t {
    return ((uint64_t)(uint32_t)blocks[seg_block_start[s]] << 32) | (uint64_t)(uint32_t)seg_len[s];
  };
  for (int s = 0; s < nseg; ++s) {
    if (!seg_is_ctx[s] || seg_len[s] <= 0) continue;
    if (seg_block_start[s + 1] <= seg_block_start[s])
      return fail(LAZY_ERR_ARG, "segment %d: %d tokens without blocks", s, seg_len[s]);
    ++readers[key_of(s)];
  }
  // 2. the shared documents, heaviest (tiles x readers) first so the longest
  //    work starts first; ties by first block for a deterministic order
  struct Doc {
    uint64_t key;
    int32_t first_seg, readers, index;
  };
  std::vector<Doc> docs;
  std::unordered_map<uint64_t, int32_t> doc_of;
  for (int s = 0; s < nseg; ++s) {
    if (!seg_is_ctx[s] || seg_len[s] <= 0) continue;
    const uint64_t k = key_of(s);
    const int32_t n = readers[k];
    if (n < min_readers || doc_of.count(k)) continue;
    doc_of[k] = -1;
    docs.push_back({k, s, n, 0});
  }
  // with min_readers 1 every request's private tokens become one more item
  // of the pass too (read once, at Delta 0: keys and query both at global
  // positions), so the split-K pass has nothing left to do
  const bool private_items = min_readers == 1;
  auto private_key = [](int s) -> uint64_t { return (1ull << 63) | (uint64_t)(uint32_t)s; };
  if (private_items)
    for (int s = 0; s < nseg; ++s) {
      if (seg_is_ctx[s] || seg_len[s] <= 0) continue;
      doc_of[private_key(s)] = -1;
      docs.push_back({private_key(s), s, 1, 0});
    }
  std::sort(docs.begin(), docs.end(), [&](const Doc& a, const Doc& b) {
    const int64_t wa = (int64_t)(seg_len[a.first_seg] + 15) / 16 * a.readers;
    const int64_t wb = (int64_t)(seg_len[b.first_seg] + 15) / 16 * b.readers;
    return wa != wb ? wa > wb : a.key < b.key;
  });
  if ((int64_t)docs.size() > docs_cap) return fail(LAZY_ERR_ARG, "docs_cap %d too small", docs_cap);
  for (size_t i = 0; i < docs.size(); ++i) doc_of[docs[i].key] = (int32_t)i;

  // 3. each shared document's tiles, at local positions (offset = local
  //    position of the tile's slot 0); a private item's at their global
  //    positions
  int64_t ndt = 0;
  for (size_t i = 0; i < docs.size(); ++i) {
    const int s = docs[i].first_seg;
    const int64_t base = seg_is_ctx[s] ? 0 : seg_pos0[s];
    doc_tile_start[i] = (int32_t)ndt;
    const int32_t L = seg_len[s];
    const int32_t nblk = (L + LAZY_BLOCK_SIZE - 1) / LAZY_BLOCK_SIZE;
    if (seg_block_start[s + 1] - seg_block_start[s] < nblk)
      return fail(LAZY_ERR_ARG, "segment %d: %d blocks for %d tokens", s, seg_block_start[s + 1] - seg_block_start[s],
                  L);
    for (int32_t b = 0; b < nblk; ++b) {
      const int64_t blk = blocks[seg_block_start[s] + b];
      if (blk < 0 || blk >= num_blocks)
        return fail(LAZY_ERR_ARG, "segment %d block %d: id %lld outside the pool", s, b, (long long)blk);
      const int32_t valid = (L - LAZY_BLOCK_SIZE * b) < LAZY_BLOCK_SIZE ? (L - LAZY_BLOCK_SIZE * b) : LAZY_BLOCK_SIZE;
      if (ndt >= doc_tiles_cap) return fail(LAZY_ERR_ARG, "doc_tiles_cap %lld too small", (long long)doc_tiles_cap);
      const int64_t off = base + (int64_t)LAZY_BLOCK_SIZE * b;
      if (off > LAZY_MAX_OFFSET) return fail(LAZY_ERR_ARG, "segment %d: offset %lld exceeds 2^24-1", s, (long long)off);
      doc_tiles_out[ndt++] = ((uint64_t)blk << 40) | ((uint64_t)off << 16) | (uint64_t)((1u << valid) - 1u);
    }
  }
  doc_tile_start[docs.size()] = (int32_t)ndt;

  // 4. chunks: a document pass of few, long documents would leave most of
  //    the chip idle.  When the pass holds fewer than `few` work items (half
  //    a resident round: 256 workgroups of the LDS pass, one per CU, or 1024
  //    waves of the per-wave pass), each document is cut into up to
  //    ceil(2 few / items) even chunks of >= kMinChunkTiles tiles, a chunk
  //    per item and its own partial slot per read; otherwise documents stay
  //    whole (every chunk adds a partial per read and per head to merge)
  const int32_t group = geom->num_q_heads / geom->num_kv_heads;
  const int32_t rb = docpass_row_blocks(geom);
  const int64_t few = docpass_uses_lds(geom) ? 256 : 1024;
  constexpr int64_t kMinChunkTiles = 32;
  int64_t items = 0;
  for (const Doc& d : docs) items += ((int64_t)d.readers * group + 16 * rb - 1) / (16 * rb);
  items *= geom->num_kv_heads;
  const int64_t want_chunks = (items > 0 && items < few) ? (2 * few + items - 1) / items : 1;
  std::vector<int32_t> nchunks(docs.size()), chunk_tiles(docs.size());
  for (size_t i = 0; i < docs.size(); ++i) {
    const int64_t nt_doc = (seg_len[docs[i].first_seg] + LAZY_BLOCK_SIZE - 1) / LAZY_BLOCK_SIZE;
    const int64_t n = std::max<int64_t>(1, std::min<int64_t>(want_chunks, nt_doc / kMinChunkTiles));
    int64_t ct = (nt_doc + n - 1) / n;
    ct = (ct + 1) & ~1LL;  // whole tile pairs
    chunk_tiles[i] = (int32_t)ct;
    nchunks[i] = (int32_t)((nt_doc + ct - 1) / ct);
  }

  // 5. reads of every shared document: (request, first slot, Delta), grouped
  //    by document (a read takes one slot per chunk); and each request's own
  //    tiles (unshared documents, then its private tokens)
  std::vector<int32_t> fill(docs.size(), 0);
  int64_t nreads = 0;
  for (size_t i = 0; i < docs.size(); ++i) {
    read_start[i] = (int32_t)nreads;
    nreads += docs[i].readers;
  }
  read_start[docs.size()] = (int32_t)nreads;
  if (nreads > reads_cap) return fail(LAZY_ERR_ARG, "reads_cap %lld too small", (long long)reads_cap);
  int64_t nt = 0, max_tiles = 0;
  int32_t max_req_reads = 0;
  for (int r = 0; r < num_reqs; ++r) {
    if (nt > INT32_MAX) return fail(LAZY_ERR_ARG, "too many tiles");
    tile_start[r] = (int32_t)nt;
    int32_t slot = 0;
    int64_t nctx = 0;
    bool seen_private = false;
    for (int s = seg_start[r]; s < seg_start[r + 1]; ++s) {
      const bool ctx = seg_is_ctx[s] != 0;
      if (ctx && seen_private) return fail(LAZY_ERR_ARG, "request %d: context segment %d after a private one", r, s);
      if (!ctx) seen_private = true;
      if (!ctx && private_items && seg_len[s] > 0) {  // the request's private item: one read at Delta 0
        const int32_t i = doc_of[private_key(s)];
        if (slot + nchunks[i] > 0xFFFF)
          return fail(LAZY_ERR_UNSUPPORTED, "request %d needs more than 65535 shared-read slots", r);
        reads_out[read_start[i] + fill[i]++] = ((uint64_t)r << 48) | ((uint64_t)slot << 32);
        slot += nchunks[i];
        continue;
      }
      if (ctx && seg_len[s] > 0) {
        auto it = doc_of.find(key_of(s));
        if (it != doc_of.end() && it->second >= 0) {
          const int32_t i = it->second;
          const Doc& d = docs[i];
          // the same physical copy everywhere it is read
          const int32_t nblk = (seg_len[s] + LAZY_BLOCK_SIZE - 1) / LAZY_BLOCK_SIZE;
          if (seg_block_start[s + 1] - seg_block_start[s] < nblk)
            return fail(LAZY_ERR_ARG, "segment %d: too few blocks", s);
          for (int32_t b = 0; b < nblk; ++b)
            if (blocks[seg_block_start[s] + b] != blocks[seg_block_start[d.first_seg] + b])
              return fail(LAZY_ERR_ARG, "segment %d: document starting at block %d has another block list", s,
                          blocks[seg_block_start[s]]);
          const int64_t delta = seg_pos0[s];
          if (delta < 0 || delta > LAZY_MAX_OFFSET)
            return fail(LAZY_ERR_ARG, "segment %d: offset %lld outside [0, 2^24)", s, (long long)delta);
          if (max_pos > 0 && kind != LAZY_ALIBI && delta >= max_pos)
            return fail(LAZY_ERR_ARG, "segment %d: document offset %lld outside the cos/sin table (max_pos %d)", s,
                        (long long)delta, max_pos);
          if (slot + nchunks[i] > 0xFFFF)
            return fail(LAZY_ERR_UNSUPPORTED, "request %d needs more than 65535 shared-read slots", r);
          reads_out[read_start[i] + fill[i]++] = ((uint64_t)r << 48) | ((uint64_t)slot << 32) | (uint64_t)delta;
          slot += nchunks[i];
          continue;
        }
      }
      const int64_t before = nt;
      st = emit_segment(kind, s, seg_len, seg_pos0, seg_is_ctx, seg_block_start, blocks, num_blocks, max_pos,
                        tiles_out, tiles_cap, nt);
      if (st != LAZY_OK) return st;
      if (ctx) nctx += nt - before;
    }
    ctx_tiles[r] = (int32_t)nctx;
    req_reads[r] = slot;
    max_req_reads = std::max(max_req_reads, slot);
    max_tiles = std::max<int64_t>(max_tiles, nt - tile_start[r]);
  }
  if (nt > INT32_MAX) return fail(LAZY_ERR_ARG, "too many tiles");
  tile_start[num_reqs] = (int32_t)nt;

  // 6. work items of the document pass: (document, first 16-row block,
  //    chunk, tiles per chunk) for every docpass_row_blocks x 16 rows of
  //    reads x query group and every chunk; a (document, chunk)'s row tiles
  //    adjacent
  int64_t nw = 0;
  for (size_t i = 0; i < docs.size(); ++i) {
    const int64_t rows = (int64_t)docs[i].readers * group;
    const int64_t n_items = (rows + 16 * rb - 1) / (16 * rb);
    for (int32_t c = 0; c < nchunks[i]; ++c)
      for (int64_t k = 0; k < n_items; ++k) {
        if (nw >= work_cap) return fail(LAZY_ERR_ARG, "work_cap %lld too small", (long long)work_cap);
        work_out[4 * nw] = (int32_t)i;
        work_out[4 * nw + 1] = (int32_t)(k * rb);
        work_out[4 * nw + 2] = c;
        work_out[4 * nw + 3] = chunk_tiles[i];
        ++nw;
      }
  }
  counts_out[0] = (int64_t)docs.size();
  counts_out[1] = nreads;
  counts_out[2] = nw;
  counts_out[3] = max_req_reads;
  counts_out[4] = nt;
  counts_out[5] = max_tiles;
  counts_out[6] = ndt;
  counts_out[7] = rb;
  return LAZY_OK;
}
