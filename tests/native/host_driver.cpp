// Drives every host-side entry point of the library (metadata, packer, tile
// builder, error text) through valid and invalid arguments.  Built from the
// library's own host source with address and undefined-behaviour sanitizers
// by tests/test_host_sanitized.py; any out-of-bounds access, use of freed
// memory, leak or undefined behaviour aborts the run.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <vector>

#include "lazy_attn.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main() {
  // positional metadata
  for (int dh : {64, 128}) {
    std::vector<double> inv(dh / 2);
    double gain = 0;
    CHECK(lazy_rope_freqs(dh, 5e5, 8.0, 8192, 32.0, 1.0, inv.data(), &gain) == LAZY_OK);
    CHECK(gain > 1.0);
    CHECK(lazy_rope_freqs(dh, 1e4, 1.0, 0, 32.0, 1.0, inv.data(), nullptr) == LAZY_OK);
    std::vector<float> table((size_t)1000 * dh);
    CHECK(lazy_rope_table(dh, inv.data(), 1000, table.data()) == LAZY_OK);
    CHECK(table[0] == 1.0f);
    float scale = 0;
    CHECK(lazy_softmax_scale(dh, 1.0, &scale) == LAZY_OK && fabsf(scale - 1.0f / sqrtf((float)dh)) < 1e-7f);
  }
  CHECK(lazy_rope_freqs(63, 1e4, 1.0, 0, 32, 1, nullptr, nullptr) == LAZY_ERR_ARG);
  CHECK(strlen(lazy_last_error()) > 0);
  CHECK(lazy_rope_table(64, nullptr, 10, nullptr) == LAZY_ERR_ARG);
  CHECK(lazy_softmax_scale(0, 1.0, nullptr) == LAZY_ERR_ARG);
  std::vector<float> slopes(71);
  CHECK(lazy_alibi_slopes(71, slopes.data()) == LAZY_OK && slopes[70] == 1.0f / 256);
  CHECK(lazy_alibi_slopes(0, slopes.data()) == LAZY_ERR_ARG);

  // packer round trip on random words, then every out-of-field value
  std::mt19937_64 rng(42);
  const int n = 100000;
  std::vector<int64_t> blk(n), off(n), b2(n), o2(n);
  std::vector<uint32_t> msk(n), m2(n);
  std::vector<uint64_t> words(n);
  for (int i = 0; i < n; ++i) {
    blk[i] = (int64_t)(rng() & 0xFFFFFF);
    off[i] = (int64_t)(rng() & 0xFFFFFF);
    msk[i] = 1 + (uint32_t)(rng() % 0xFFFF);
  }
  CHECK(lazy_pack_tiles(blk.data(), off.data(), msk.data(), n, words.data()) == LAZY_OK);
  CHECK(lazy_unpack_tiles(words.data(), n, b2.data(), o2.data(), m2.data()) == LAZY_OK);
  CHECK(blk == b2 && off == o2 && msk == m2);
  CHECK(lazy_unpack_tiles(words.data(), n, nullptr, nullptr, nullptr) == LAZY_OK);
  int64_t bad_blk = 1 << 24, ok = 0, bad_off = -1;
  uint32_t m0 = 0, m1 = 1, mbig = 0x10000;
  uint64_t w = 0;
  CHECK(lazy_pack_tiles(&bad_blk, &ok, &m1, 1, &w) == LAZY_ERR_ARG);
  CHECK(lazy_pack_tiles(&ok, &bad_off, &m1, 1, &w) == LAZY_ERR_ARG);
  CHECK(lazy_pack_tiles(&ok, &ok, &m0, 1, &w) == LAZY_ERR_ARG);
  CHECK(lazy_pack_tiles(&ok, &ok, &mbig, 1, &w) == LAZY_ERR_ARG);
  CHECK(lazy_pack_tiles(nullptr, nullptr, nullptr, -1, nullptr) == LAZY_ERR_ARG);

  // tile builder: random layouts with exact and short capacities
  for (int trial = 0; trial < 200; ++trial) {
    const int R = 1 + (int)(rng() % 6);
    std::vector<int32_t> seg_start{0}, seg_len, seg_bs{0}, blocks;
    std::vector<int64_t> seg_pos0;
    std::vector<uint8_t> seg_ctx;
    int64_t tiles = 0;
    for (int r = 0; r < R; ++r) {
      const int nseg = (int)(rng() % 5);
      int64_t pos = 0;
      for (int s = 0; s < nseg; ++s) {
        const int L = (int)(rng() % 70);
        const bool ctx = s + 1 < nseg;
        seg_len.push_back(L);
        seg_pos0.push_back(pos);
        seg_ctx.push_back(ctx ? 1 : 0);
        const int nb = (L + 15) / 16;
        for (int b = 0; b < nb; ++b) blocks.push_back((int32_t)(rng() % 500));
        seg_bs.push_back((int32_t)blocks.size());
        tiles += nb;
        pos += L;
      }
      seg_start.push_back((int32_t)seg_len.size());
    }
    if (blocks.empty()) blocks.push_back(0);
    std::vector<uint64_t> out(tiles + 1);
    std::vector<int32_t> tstart(R + 1), nctx(R);
    const int32_t* bl = blocks.data();
    CHECK(lazy_build_tiles(trial % 3, R, seg_start.data(), seg_len.data(), seg_pos0.data(), seg_ctx.data(),
                           seg_bs.data(), bl, 500, 0, out.data(), tiles, tstart.data(), nctx.data()) == LAZY_OK);
    CHECK(tstart[R] == tiles);
    {  // documents closed to whole tile pairs: every request's context tile count even
      std::vector<uint64_t> outp(tiles + seg_len.size() + 1);
      CHECK(lazy_build_tiles_paired(trial % 3, R, seg_start.data(), seg_len.data(), seg_pos0.data(), seg_ctx.data(),
                                    seg_bs.data(), bl, 500, 0, outp.data(), (int64_t)outp.size(), tstart.data(),
                                    nctx.data()) == LAZY_OK);
      for (int r = 0; r < R; ++r) CHECK(nctx[r] % 2 == 0);
      CHECK(lazy_build_tiles(trial % 3, R, seg_start.data(), seg_len.data(), seg_pos0.data(), seg_ctx.data(),
                             seg_bs.data(), bl, 500, 0, out.data(), tiles, tstart.data(), nctx.data()) == LAZY_OK);
    }
    if (tiles > 0) {
      CHECK(lazy_build_tiles(trial % 3, R, seg_start.data(), seg_len.data(), seg_pos0.data(), seg_ctx.data(),
                             seg_bs.data(), bl, 500, 0, out.data(), tiles - 1, tstart.data(), nctx.data()) ==
            LAZY_ERR_ARG);
      // a pool smaller than some block id is refused, never read past
      bool beyond = false;
      for (int32_t b : blocks) beyond = beyond || b >= 100;
      CHECK(lazy_build_tiles(trial % 3, R, seg_start.data(), seg_len.data(), seg_pos0.data(), seg_ctx.data(),
                             seg_bs.data(), bl, 100, 0, out.data(), tiles, tstart.data(), nctx.data()) ==
            (beyond ? LAZY_ERR_ARG : LAZY_OK));
      // a cos/sin table shorter than some rotary document offset is refused
      int64_t far = -1;
      for (int r = 0; r < R; ++r)
        for (int s = seg_start[r]; s < seg_start[r + 1]; ++s)
          if (seg_ctx[s] && seg_len[s] > 0) far = far > seg_pos0[s] ? far : seg_pos0[s];
      if (far > 0 && trial % 3 != LAZY_ALIBI)
        CHECK(lazy_build_tiles(trial % 3, R, seg_start.data(), seg_len.data(), seg_pos0.data(), seg_ctx.data(),
                               seg_bs.data(), bl, 500, (int32_t)far, out.data(), tiles, tstart.data(),
                               nctx.data()) == LAZY_ERR_ARG);
    }
  }
  CHECK(lazy_build_tiles(9, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 0, nullptr, 0, nullptr,
                         nullptr) == LAZY_ERR_ARG);

  // document-major plan: requests drawing documents from a shared pool, generous and short capacities
  lazy_geom geom{32, 8, 128, 16, LAZY_BF16};
  for (int trial = 0; trial < 100; ++trial) {
    const int R = 1 + (int)(rng() % 8), pool = 1 + (int)(rng() % 6);
    std::vector<int32_t> doc_len(pool), doc_b0(pool);
    int32_t nb = 0;
    for (int d = 0; d < pool; ++d) {
      doc_len[d] = 1 + (int)(rng() % 600);
      doc_b0[d] = nb;
      nb += (doc_len[d] + 15) / 16;
    }
    std::vector<int32_t> seg_start{0}, seg_len, seg_bs{0}, blocks;
    std::vector<int64_t> seg_pos0;
    std::vector<uint8_t> seg_ctx;
    for (int r = 0; r < R; ++r) {
      int64_t pos = 0;
      const int nd = (int)(rng() % 5);
      for (int k = 0; k < nd; ++k) {
        const int d = (int)(rng() % pool);
        seg_len.push_back(doc_len[d]);
        seg_pos0.push_back(pos);
        seg_ctx.push_back(1);
        for (int b = 0; b < (doc_len[d] + 15) / 16; ++b) blocks.push_back(doc_b0[d] + b);
        seg_bs.push_back((int32_t)blocks.size());
        pos += doc_len[d];
      }
      seg_len.push_back(3);
      seg_pos0.push_back(pos);
      seg_ctx.push_back(0);
      blocks.push_back(nb++);
      seg_bs.push_back((int32_t)blocks.size());
      seg_start.push_back((int32_t)seg_len.size());
    }
    const int64_t cap = (int64_t)blocks.size() + 1, docs_cap = (int64_t)seg_len.size() + 1;
    const int64_t work_cap = 4096;
    std::vector<uint64_t> tiles(cap), dtiles(cap), reads(docs_cap);
    std::vector<int32_t> tstart(R + 1), nctx(R), dstart(docs_cap + 1), rstart(docs_cap + 1), rreads(R), work(4 * work_cap);
    std::vector<int64_t> counts(8);
    for (int shortcap = 0; shortcap < 2; ++shortcap) {
      const lazy_status st = lazy_build_shared_plan(
          &geom, trial % 3, R, seg_start.data(), seg_len.data(), seg_pos0.data(), seg_ctx.data(), seg_bs.data(),
          blocks.data(), nb, 0, 2, tiles.data(), shortcap ? 0 : cap, tstart.data(), nctx.data(), dtiles.data(), cap,
          dstart.data(), rstart.data(), (int32_t)docs_cap, reads.data(), docs_cap, rreads.data(), work.data(),
          shortcap ? 0 : work_cap, counts.data());
      if (shortcap) {
        CHECK(st == LAZY_ERR_ARG);
      } else {
        CHECK(st == LAZY_OK);
        CHECK(counts[4] <= cap && counts[6] <= cap && counts[1] <= docs_cap && counts[2] <= work_cap);
      }
    }
  }
  printf("host driver: all checks passed\n");
  return 0;
}
