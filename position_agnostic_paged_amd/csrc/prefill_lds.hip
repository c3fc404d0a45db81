// LDS-staged prefill over a position-agnostic paged cache (bf16, gfx950).
//
// Same computation as the per-wave prefill, organised as the pages' prefill
// kernel (LazyAttention notes, papernotes.org, "Key designs": the K tile is
// staged in shared memory and rotated there by the document offset Delta
// before the matrix products), adapted to CDNA4:
//
//   * a workgroup = NW waves x RB blocks of 16 GQA-packed query rows of one
//     (request, KV head); all waves consume the same tile pairs;
//   * each tile pair (K 2 x 16 x dh, V 2 x dh x 16, plus the two cos/sin
//     rows of the pair's document offsets) is copied once per workgroup
//     from HBM into LDS with direct global->LDS loads (no registers), into a
//     ring of kStages buffers that fills the 160 KiB LDS, so kStages-3 pairs
//     are in flight while one pair is rotated, the next one's scores are
//     computed and the one before it is consumed (the copies are
//     latency-bound: bytes in flight set the rate);
//   * once a pair has landed, the workgroup rotates its context K rows in
//     place by R_Delta (fp32 arithmetic, rounded back to bf16), turning the
//     position-agnostic R_j k into R_(Delta+j) k; the query stays at its
//     global position in registers for the whole loop;
//   * LDS rows are XOR-swizzled at 16-byte granularity so the per-lane
//     fragment reads (16 B of a K row, 16 B of a V channel row) are free of
//     bank conflicts;
//   * the softmax is trimmed for the matrix cores: pairs of two full
//     document tiles (the bulk of a long context) skip masking; the row max
//     is taken on raw scores against a per-row threshold, so the cross-lane
//     reduction and the rescale only run when some row's maximum grows by
//     more than 2^LAZY_RESCALE_SLACK; the scale folds into the exponent's
//     FMA; row sums come from one extra MFMA against a ones operand (the
//     sum of exactly the bf16 weights that multiply V);
//   * the wave raises its issue priority over its run of P V products, so
//     they go out back to back while the other wave of the SIMD fills the
//     matrix core's shadow with vector work;
//   * a pair's two tile words are decoded once, when its copies are issued,
//     into a small header in its stage buffer (the CU's one scalar unit
//     serves all eight waves);
//   * the two waves sharing a SIMD take each iteration's halves in opposite
//     orders, so one's matrix products overlap the other's vector, scalar
//     and LDS work between the same two barriers.
#include <atomic>

#include "attn_common.hpp"

namespace lazy {

#ifndef LAZY_PREFILL_WAVES
#define LAZY_PREFILL_WAVES 8  // waves per workgroup: 8 = two per SIMD, 2 x 16 rows each (4 = one per SIMD,
                              // 4 x 16 rows: spills at dh 128, the rescale keeps the accumulators in VGPRs)
#endif
constexpr int kPrefillWaves = LAZY_PREFILL_WAVES;
// The document pass's ring: LAZY_DOCPASS_STAGES tile pairs (four: 64 KiB at
// dh 128, so two workgroups share a CU and one's ring fill and barriers
// overlap the other's work), copied with the streaming hint (mixed 70B
// decode call 0.286 -> 0.276 ms), and a register cap for
// LAZY_DOCPASS_LDS_WPE waves per SIMD (both workgroups resident).
#ifndef LAZY_DOCPASS_STAGES
#define LAZY_DOCPASS_STAGES 4
#endif
#ifndef LAZY_DOCPASS_LDS_WPE
#define LAZY_DOCPASS_LDS_WPE (LAZY_DOCPASS_LDS_WAVES / 2)
#endif
constexpr int kLdsBytes = 160 * 1024;    // LDS of one CU, all of it for the ring

// Wait until at most N vector-memory operations of this wave are outstanding
// and, before a bare s_barrier, all of its LDS and scalar-memory operations
// (lgkmcnt 0): the wave's LDS writes (rotated K rows, pair headers) must have
// completed before other waves read them after the barrier.  The direct
// global->LDS copies count on vmcnt only, so the later pairs' copies stay in
// flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0x0 << 8) | ((N >> 4) << 14));
}

// Only this wave's LDS and scalar-memory operations (vmcnt left at its maximum).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14)); }

// Wait until at most n stages of L copies each are outstanding (n <= MAXN),
// then for lgkmcnt 0 (every caller is followed by a barrier).
template <int L, int MAXN>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (MAXN > 0) {
    if (n >= MAXN) {
      wait_vmcnt_lgkm0<MAXN * L>();
      return;
    }
    wait_stages<L, MAXN - 1>(n);
  } else {
    wait_vmcnt_lgkm0<0>();
  }
}

// ROT: each stage's K tiles are rotated in LDS (two cos/sin rows per stage);
// QROT: the query is rotated per document (one cos/sin row per stage, the
// pair's); RESERVE bytes after the ring hold the waves' raw query rows.
template <int DH, bool ROT, int NW, int MAXS = 10, bool QROT = false, int RESERVE = 0>
struct StageGeom {
  static constexpr int kTile = kBlock * DH * 2;      // bytes of one 16 x dh bf16 tile
  static constexpr int kChunksPerRow = DH / 8;       // 16-byte chunks in a K row
  static constexpr int kK = 0;                       // two K tiles
  static constexpr int kV = 2 * kTile;               // two V tiles
  static constexpr int kCS = 4 * kTile;              // cos/sin rows (fp32 [dh] each)
  static constexpr int kCsRows = ROT ? 2 : (QROT ? 1 : 0);
  static constexpr int kHdr = kCS + kCsRows * DH * 4;  // the pair's decoded tile words (PairHdr)
  static constexpr int kBytes = kHdr + 32;
  static constexpr int kKChunks = 2 * kTile / 16;    // 16-B chunks of the K pair (same for V)
  static constexpr int kCopies = 2 * kKChunks / (NW * 64);  // K + V copies per thread
  static constexpr int kLoads = kCopies + (kCsRows > 0 ? 1 : 0);  // copies per wave per stage
  static constexpr int kRing = kLdsBytes - RESERVE;
  static constexpr int kStages = (kRing / kBytes) < MAXS ? (kRing / kBytes) : MAXS;
  static constexpr int kReserve = kStages * kBytes;  // offset of the reserved bytes
  static constexpr int kLdsTotal = kStages * kBytes + RESERVE;
  static_assert(!(ROT && QROT), "one rotation side");
  // Pairs past the consumed one that each iteration waits for: with the K
  // rotation, pair p + 2 (rotated during iteration p); without it, pair
  // p + 1 (its scores end iteration p), which leaves one more stage in flight
  // and lets a ring of four stages work.
  static constexpr int kAhead = ROT ? 2 : 1;
  // every wave issues the same number of copies (the counted waits rely on
  // it) and no wave's 64 chunks straddle the K / V boundary
  static_assert(kCopies >= 1 && (2 * kKChunks) % (NW * 64) == 0 && kKChunks % 64 == 0, "stage copy shape");
  static_assert(kStages >= 3 + kAhead && (kStages - 1 - kAhead) * kLoads < 64, "ring depth");
  // rotation items: 16 rows x dh/8 items (4 rotation pairs each) per tile
  static constexpr int kRotItems = kBlock * DH / 8;
  static_assert(kRotItems % 64 == 0, "rotation items per wave");
};

typedef const __attribute__((address_space(4))) uint64_t* const_words;

// Raw tile words of one pair (the second is 0 -- an empty tile -- past the
// split's end).
struct PairWords {
  uint64_t w0, w1;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A pair's tile words decoded once, when its copies are issued, and kept in
// its stage buffer for the rotation and the softmax: 32 bytes,
//   [0] mask0 | mask1 << 16 (after the guards: a dropped tile has mask 0)
//   [1] [2] the two tiles' word offsets (token position of the first slot)
//   [3] bit 0 / 1: tile 0 / 1 is private; bit 2: both tiles full document tiles
//   [4] [5] the rotation offsets Delta (0 where nothing is rotated)
// Every wave would otherwise decode each pair three times on the CU's one
// scalar unit.
constexpr uint32_t kHdrPriv0 = 1u, kHdrPriv1 = 2u, kHdrFull = 4u;

// K row swizzle: the 16-byte chunk q of row t of tile x sits at chunk
// position q ^ key; tile 1 uses keys disjoint from tile 0's for the rows one
// fragment read touches together.
template <int DH>
__device__ __forceinline__ int k_key(int t, int x) {
  return (t ^ (4 * x)) % (DH / 8);
}

// Workgroup -> work unit.  The workgroups of one (request, KV head, split)
// -- its row tiles -- read the same K/V tiles, so they are placed on one XCD
// (dispatch deals workgroups round-robin over the 8 XCDs, each with its own
// L2) and dispatched close together: the second reader finds the tiles in
// L2.  A 1-D grid of units x row_tiles workgroups; with a unit count that is
// not a multiple of 8 the plain order is used.
constexpr int kXcds = 8;

__device__ __forceinline__ void xcd_unit(int wg, int num_wgs, int splits, int hkv, int row_tiles, int& req, int& kvh,
                                         int& split, int& row_tile) {
  const int units = num_wgs / row_tiles;
  int u, t;
  if (units % kXcds == 0) {
    const int k = wg / kXcds;
    t = k % row_tiles;
    u = (k / row_tiles) * kXcds + wg % kXcds;
  } else {
    u = wg / row_tiles;
    t = wg % row_tiles;
  }
  split = u % splits;
  kvh = (u / splits) % hkv;
  req = u / (splits * hkv);
  row_tile = t;
}

template <int DH, int KIND, bool DEFER, int RB, int NW, int MAXS = 10, bool NT = false, bool QROT = false>
struct LdsPrefill {
  using F8 = bf16x8;
  using F4 = bf16x4;
  static constexpr int NC = DH / 32;  // contraction chunks of QK^T
  static constexpr int NV = DH / 16;  // 16-channel blocks of the output
  // kRot: K rotated by Delta in LDS per pair; kQRot: the query rotated by
  // -Delta once per document (the tile lists keep each pair in one document)
  static constexpr bool kRot = (KIND != kAlibi) && DEFER && !QROT;
  static constexpr bool kQRot = (KIND != kAlibi) && DEFER && QROT;
  static constexpr int kQBytes = RB * NC * 64 * 16;  // one wave's raw query fragments
  using SG = StageGeom<DH, kRot, NW, MAXS, kQRot, kQRot ? NW * kQBytes : 0>;
  static constexpr int S = SG::kStages;

  const AttnArgs& a;
  unsigned char* lds;
  int tid, lane, wave, kvh, sb, se, nctx, npairs;
  // The tile table is read-only for the kernel's lifetime, so it is read
  // through the constant address space: scalar loads, counted apart from the
  // stage copies.
  const_words words;
  uint32_t copy_off[SG::kCopies];  // per-lane byte offset of each stage copy in its tile

  __device__ __forceinline__ void init_copies() {
#pragma unroll
    for (int i = 0; i < SG::kCopies; ++i) {
      const int cb = (i * NW + wave) * 64;  // wave-uniform first chunk
      const bool is_v = cb >= SG::kKChunks;
      const int cv = (is_v ? cb - SG::kKChunks : cb) + lane;
      const int x = cv / (SG::kTile / 16);
      const int cc = cv % (SG::kTile / 16);
      int elem;
      if (!is_v) {
        const int row = cc / SG::kChunksPerRow, pos = cc % SG::kChunksPerRow;
        elem = row * DH + (pos ^ k_key<DH>(row, x)) * 8;
      } else {  // V rows are channels of 16 tokens = 2 chunks
        const int row = cc >> 1, pos = cc & 1;
        elem = row * kBlock + (pos ^ ((row >> 3) & 1)) * 8;
      }
      copy_off[i] = (uint32_t)elem * 2u;
    }
  }

  // Stage buffers are addressed relative to the buffer of pair base_q, whose
  // byte offset base_off the loop keeps in one scalar register: pair q
  // (base_q <= q < base_q + S) sits kBytes (q - base_q) further on, wrapped
  // once.  A modulo per use would be strength-reduced by the compiler into
  // two terms, each added to every per-lane LDS address.
  uint32_t base_off = 0;
  int base_q = 0;
  __device__ __forceinline__ uint32_t stage_off(int q) const {
    const uint32_t o = base_off + (uint32_t)(q - base_q) * SG::kBytes;
    return o >= (uint32_t)(S * SG::kBytes) ? o - (uint32_t)(S * SG::kBytes) : o;
  }
  __device__ __forceinline__ unsigned char* stage(int q) const { return lds + stage_off(q); }

  __device__ __forceinline__ PairWords load_words(int q) const {
    PairWords pw{0ull, 0ull};
    if (q < npairs) {
      const int ia = sb + 2 * q;
      pw.w0 = words[ia];
      if (ia + 1 < se) pw.w1 = words[ia + 1];
    }
    return pw;
  }

  // tile words of a pair, decoded with the device-side guards
  __device__ __forceinline__ void pair_meta(int q, const PairWords& pw, TileMeta (&mt)[2], int (&delta)[2],
                                            bool (&priv)[2]) const {
    const int ia = sb + 2 * q;
    mt[0] = unpack_word(pw.w0);
    mt[1] = unpack_word(pw.w1);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      priv[x] = ia + x >= nctx;
      if (mt[x].block >= a.num_blocks || mt[x].block < 0) {  // never dereference outside the pool
        mt[x].block = 0;
        mt[x].mask = 0u;
      }
      delta[x] = (kRot && !priv[x]) ? mt[x].offset : 0;
      if (kRot && delta[x] >= a.max_pos) {  // outside the table: drop the tile
        mt[x].mask = 0u;
        delta[x] = 0;
      }
    }
    if (kQRot) {
      // one rotation per pair: tile 0's document offset (0 for private
      // tokens, whose keys and query both sit at global positions)
      int d = priv[0] ? 0 : mt[0].offset;
      if (d >= a.max_pos) {  // outside the table: drop the pair
        mt[0].mask = mt[1].mask = 0u;
        d = 0;
      }
      delta[0] = d;
      delta[1] = 0;
    }
  }

  // copy pair q into its stage buffer (every wave issues SG::kLoads copies)
  __device__ __forceinline__ void issue(int q, const PairWords& pw) const {
    TileMeta mt[2];
    int delta[2];
    bool priv[2];
    pair_meta(q, pw, mt, delta, priv);
    unsigned char* st = stage(q);
#pragma unroll
    for (int i = 0; i < SG::kCopies; ++i) {
      // chunk ci of the stage's K pair, then V pair; the LDS slot of a copy
      // is the wave's base plus 16 B per lane, i.e. stage offset 16 * ci
      const int cb = (i * NW + wave) * 64;
      const bool is_v = cb >= SG::kKChunks;
      const int x = (is_v ? cb - SG::kKChunks : cb) / (SG::kTile / 16);
      const int blk = x ? mt[1].block : mt[0].block;
      const char* base = reinterpret_cast<const char*>(is_v ? a.v_cache : a.k_cache) +
                         ((int64_t)blk * a.hkv + kvh) * (int64_t)(kBlock * DH * 2);
      __builtin_amdgcn_global_load_lds(base + copy_off[i], st + cb * 16, 16, 0, NT ? kCopyAuxStream : 0);
    }
    if constexpr (SG::kCsRows > 0) {
      // the cos/sin rows (two: the tiles' offsets; one: the pair's): DH/4
      // chunks each; wave w copies its share (lane-masked)
      constexpr int kCsChunks = SG::kCsRows * (DH / 4);
      constexpr int kPerWave = kCsChunks / NW;
      static_assert(kPerWave >= 1 && kCsChunks <= 64, "cos/sin copy shape");
      if (lane >= wave * kPerWave && lane < (wave + 1) * kPerWave) {
        const int x = lane / (DH / 4);
        const int j = lane % (DH / 4);
        const int d = x ? delta[1] : delta[0];
        const float* src = a.cos_sin + (int64_t)d * DH + j * 4;  // a table is required (host checks)
        __builtin_amdgcn_global_load_lds(src, st + SG::kCS, 16, 0, 0);
      }
    }
    // the decoded words for the later stages of this pair (one lane writes;
    // read after at least three more barriers)
    if (wave == 0 && lane == 0) {
      const bool full = KIND != kAlibi && (mt[0].mask & mt[1].mask) == 0xFFFFu && !priv[0] && !priv[1];
      const u32x4 h = {mt[0].mask | (mt[1].mask << 16), (uint32_t)mt[0].offset, (uint32_t)mt[1].offset,
                       (priv[0] ? kHdrPriv0 : 0u) | (priv[1] ? kHdrPriv1 : 0u) | (full ? kHdrFull : 0u)};
      const u32x2 d = {(uint32_t)delta[0], (uint32_t)delta[1]};
      *reinterpret_cast<u32x4*>(st + SG::kHdr) = h;
      *reinterpret_cast<u32x2*>(st + SG::kHdr + 16) = d;
    }
  }

  // the header words of pair q (broadcast LDS reads; made uniform by the caller)
  __device__ __forceinline__ u32x4 read_hdr(int q) const {
    return *reinterpret_cast<const u32x4*>(stage(q) + SG::kHdr);
  }
  __device__ __forceinline__ u32x2 read_deltas(int q) const {
    return *reinterpret_cast<const u32x2*>(stage(q) + SG::kHdr + 16);
  }

  // R_Delta applied in place to the context K rows of a landed pair, in two
  // halves so the LDS reads can be issued early and their latency hidden
  // behind the matrix products: rot_load reads this thread's items, rot_store
  // rotates them (fp32) and writes them back.  An item is 4 rotation pairs of
  // one row (half-split: dims 4u..4u+3 with their partners dh/2 away;
  // interleaved: dims 8u..8u+7); a pair of tiles has 4 dh items over the
  // workgroup's threads.  Tiles with Delta = 0 (private tokens, a document at
  // position 0, dropped tiles) are already at their global positions.
  static constexpr int kRI = (2 * SG::kRotItems + NW * 64 - 1) / (NW * 64);  // items per thread
  struct RotItem {
    F8 v;  // half-split: [lo dims | hi dims]; interleaved: the 8 dims
    f32x4 c, s;
    uint32_t o_lo, o_hi;  // byte offsets (o_hi unused for interleaved)
    bool on;
  };
  struct RotWork {
    RotItem it[kRI];
  };

  __device__ __forceinline__ RotWork rot_load(int q, const int (&delta)[2]) const {
    RotWork rw;
#pragma unroll
    for (int k = 0; k < kRI; ++k) rw.it[k].on = false;
    if (!kRot) return rw;
    const uint32_t st = stage_off(q);
#pragma unroll
    for (int k = 0; k < kRI; ++k) {
      RotItem& w = rw.it[k];
      const int wbase = (k * NW + wave) * 64;  // wave-uniform
      if (wbase >= 2 * SG::kRotItems) continue;
      const int x = wbase / SG::kRotItems;
      if ((x ? delta[1] : delta[0]) == 0) continue;
      w.on = true;
      const int i = wbase % SG::kRotItems + lane;
      const int t = i / (DH / 8), u = i % (DH / 8);
      const float* cs = reinterpret_cast<const float*>(lds + st + SG::kCS) + x * DH;
      const uint32_t row = st + SG::kK + x * SG::kTile + t * (DH * 2);
      const int key = k_key<DH>(t, x);
      w.c = *reinterpret_cast<const f32x4*>(cs + 4 * u);
      w.s = *reinterpret_cast<const f32x4*>(cs + DH / 2 + 4 * u);
      if (KIND == kHalf) {
        w.o_lo = row + ((((4 * u) / 8) ^ key) << 4) + ((u & 1) << 3);
        w.o_hi = row + ((((4 * u + DH / 2) / 8) ^ key) << 4) + ((u & 1) << 3);
        const F4 lo = *reinterpret_cast<const F4*>(lds + w.o_lo), hi = *reinterpret_cast<const F4*>(lds + w.o_hi);
        w.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        w.o_lo = row + ((u ^ key) << 4);
        w.o_hi = 0;
        w.v = *reinterpret_cast<const F8*>(lds + w.o_lo);
      }
    }
    return rw;
  }

  __device__ __forceinline__ void rot_store(const RotWork& rw) const {
#pragma unroll
    for (int k = 0; k < kRI; ++k) {
      const RotItem& w = rw.it[k];
      if (!w.on) continue;
      if (KIND == kHalf) {
        F4 nlo, nhi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x1 = (float)w.v[j], x2 = (float)w.v[4 + j];
          nlo[j] = (bf16)(x1 * w.c[j] - x2 * w.s[j]);
          nhi[j] = (bf16)(x2 * w.c[j] + x1 * w.s[j]);
        }
        *reinterpret_cast<F4*>(lds + w.o_lo) = nlo;
        *reinterpret_cast<F4*>(lds + w.o_hi) = nhi;
      } else {
        F8 nv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x1 = (float)w.v[2 * j], x2 = (float)w.v[2 * j + 1];
          nv[2 * j] = (bf16)(x1 * w.c[j] - x2 * w.s[j]);
          nv[2 * j + 1] = (bf16)(x2 * w.c[j] + x1 * w.s[j]);
        }
        *reinterpret_cast<F8*>(lds + w.o_lo) = nv;
      }
    }
  }

  __device__ __forceinline__ void rotate_stage(int q) const {
    const u32x2 d = read_deltas(q);
    const int delta[2] = {uniform((int)d[0]), uniform((int)d[1])};
    rot_store(rot_load(q, delta));
  }

  // The wave's raw query fragments (global positions) in its reserved LDS
  // bytes, and their rotation by -Delta of pair q's document into qw, with
  // the pair's cos/sin row from its stage (the decode's query rotation,
  // applied once per document change).
  __device__ __forceinline__ uint32_t q_slot(int b, int c) const {
    return (uint32_t)(SG::kReserve + wave * kQBytes + ((b * NC + c) * 64 + lane) * 16);
  }
  __device__ __forceinline__ void store_q(const F8 (&qr)[RB][NC]) const {
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int c = 0; c < NC; ++c) *reinterpret_cast<F8*>(lds + q_slot(b, c)) = qr[b][c];
  }
  __device__ __forceinline__ void rotate_q(int q, F8 (&qw)[RB][NC]) const {
    const float* cs = reinterpret_cast<const float*>(stage(q) + SG::kCS);
    const int g = lane >> 4;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if (KIND == kHalf) {
#pragma unroll
        for (int c = 0; c < NC / 2; ++c) {
          const F8 lo = *reinterpret_cast<const F8*>(lds + q_slot(b, c));
          const F8 hi = *reinterpret_cast<const F8*>(lds + q_slot(b, c + NC / 2));
          const int k0 = 32 * c + 8 * g;
          const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs + k0), c1 = *reinterpret_cast<const f32x4*>(cs + k0 + 4);
          const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs + DH / 2 + k0);
          const f32x4 s1 = *reinterpret_cast<const f32x4*>(cs + DH / 2 + k0 + 4);
          F8 nlo, nhi;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float co = t < 4 ? c0[t & 3] : c1[t & 3], si = t < 4 ? s0[t & 3] : s1[t & 3];
            const float x1 = (float)lo[t], x2 = (float)hi[t];
            nlo[t] = (bf16)(x1 * co + x2 * si);
            nhi[t] = (bf16)(x2 * co - x1 * si);
          }
          qw[b][c] = nlo;
          qw[b][c + NC / 2] = nhi;
        }
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const F8 x = *reinterpret_cast<const F8*>(lds + q_slot(b, c));
          const int k0 = 16 * c + 4 * g;
          const f32x4 co = *reinterpret_cast<const f32x4*>(cs + k0);
          const f32x4 si = *reinterpret_cast<const f32x4*>(cs + DH / 2 + k0);
          F8 n;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float x1 = (float)x[2 * u], x2 = (float)x[2 * u + 1];
            n[2 * u] = (bf16)(x1 * co[u] + x2 * si[u]);
            n[2 * u + 1] = (bf16)(x2 * co[u] - x1 * si[u]);
          }
          qw[b][c] = n;
        }
      }
    }
  }

  // Raw scores of a pair's two tiles (K rows at their global positions):
  // s[h][b][j] = score of query row r of block b against the key whose
  // product row the lane's koff[h] selects.
  __device__ __forceinline__ void scores(const unsigned char* st, const uint32_t (&koff)[2][NC],
                                         const F8 (&qr)[RB][NC], f32x4 (&s)[2][RB]) const {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      F8 kf[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) kf[c] = *reinterpret_cast<const F8*>(st + koff[h][c]);
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qr[b][c], z, 0, 0, 0);
        s[h][b] = z;
      }
    }
  }
};

// The pipelined loop over a unit's tile pairs, shared by the prefill and the
// document pass: every wave of the workgroup copies (and, with deferred
// rotation, rotates) the pairs; a wave with rows (has_rows) also runs its RB
// blocks of 16 query rows qr against them.  Returns the wave's unnormalised
// accumulators, row sums (replicated in the four registers) and log2-domain
// reference maxima.  qp is each row's query position and slope_raw its ALiBi
// slope over the softmax scale (masking: causal against private tiles, the
// bias against every tile).
template <int DH, int KIND, bool DEFER, int RB, int NW, int MAXS, bool NT, bool QROT>
__device__ __forceinline__ void lds_attend(LdsPrefill<DH, KIND, DEFER, RB, NW, MAXS, NT, QROT>& pl,
                                           const typename LdsPrefill<DH, KIND, DEFER, RB, NW, MAXS, NT, QROT>::F8 (&qr_in)[RB][DH / 32],
                                           const int (&qp)[RB], const float (&slope_raw)[RB], bool has_rows,
                                           f32x4 (&acc)[RB][DH / 16], f32x4 (&lsum)[RB], float (&m_run)[RB]) {
  using P = LdsPrefill<DH, KIND, DEFER, RB, NW, MAXS, NT, QROT>;
  using F8 = typename P::F8;
  constexpr int NC = P::NC;
  constexpr int NV = P::NV;
  using SG = typename P::SG;
  constexpr int S = P::S;
  const AttnArgs& a = pl.a;
  // ids through the intrinsics again (measured: fewer registers than the copies in pl)
  const int lane = __builtin_amdgcn_workitem_id_x() & 63;
  const int wave = uniform((int)__builtin_amdgcn_workitem_id_x() >> 6);
  const int npairs = pl.npairs;
  const int r = lane & 15, g = lane >> 4;
  // the query fragments the products use; with the per-document query
  // rotation, the raw ones (global positions) wait in LDS and these hold
  // them rotated by -Delta of the current document
  F8 qr[RB][NC];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int c = 0; c < NC; ++c) qr[b][c] = qr_in[b][c];
  if constexpr (P::kQRot) {
    if (has_rows) pl.store_q(qr);
  }
  int dq_cur = 0;  // the query's current rotation (0: raw)

  // Fragment offsets inside a stage (loop-invariant).  K product h, chunk c:
  // row r of the product is key (tile r/8, token 8 ((r/4)%2) + 4h + r%4), so
  // each lane's eight scores s[h][b][j] are the consecutive tokens
  // 8 (g%2) + 4h + j of tile g/2 -- the slots of the lane's single 16-byte V
  // read (channel row 16n + r of tile g/2).
  uint32_t koff[2][NC];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int x = r >> 3;
    const int t = 8 * ((r >> 2) & 1) + 4 * h + (r & 3);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      koff[h][c] = SG::kK + x * SG::kTile + t * (DH * 2) + (((4 * c + g) ^ k_key<DH>(t, x)) << 4);
  }
  const uint32_t voff = SG::kV + (g >> 1) * SG::kTile + r * 32 + (((g & 1) ^ ((r >> 3) & 1)) << 4);

  float negm[RB], thr[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int n = 0; n < NV; ++n) acc[b][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    lsum[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[b] = -INFINITY;  // log2-domain reference max
    negm[b] = 0.f;         // -m_run (0 while m_run is -inf)
    thr[b] = -INFINITY;    // raw score above which the reference must move
  }
  const float sl = a.scale_log2;
  F8 ones;
#pragma unroll
  for (int t = 0; t < 8; ++t) ones[t] = (bf16)1.f;

  // prologue: S - 1 pairs in flight; pairs 0 .. kA - 1 landed (and, with
  // the K rotation, rotated); scores of pair 0
  constexpr int kA = SG::kAhead;
#pragma unroll
  for (int q = 0; q < S - 1; ++q)
    if (q < npairs) pl.issue(q, pl.load_words(q));
  wait_stages<SG::kLoads, S - 1 - kA>(min(S - 1 - kA, npairs - kA));
  asm volatile("s_barrier" ::: "memory");
  // Tile words of the pair to copy next travel through scalar registers, read
  // one iteration ahead; the later stages use the pair's decoded header,
  // likewise read one iteration ahead (pair p + 1 for the softmax, p + 3 for
  // the rotation).
  PairWords wi = pl.load_words(S - 1);
  u32x4 hc;
  int dr[2] = {0, 0};
  {
    const u32x4 h = pl.read_hdr(0);
#pragma unroll
    for (int k = 0; k < 4; ++k) hc[k] = (uint32_t)uniform((int)h[k]);
  }
  if constexpr (P::kRot) {
    pl.rotate_stage(0);
    if (1 < npairs) pl.rotate_stage(1);
    const u32x2 d = pl.read_deltas(2);
    dr[0] = uniform((int)d[0]);
    dr[1] = uniform((int)d[1]);
  }
  if constexpr (P::kQRot) {
    // the first pair's document (its stage landed before the barrier above;
    // the query's own LDS writes are this wave's and need no barrier)
    const int d0 = uniform((int)pl.read_deltas(0)[0]);
    if (has_rows && d0 != 0) pl.rotate_q(0, qr);
    dq_cur = d0;
  }
  wait_lgkm0();  // the rotated rows of pairs 0 and 1 are written before the barrier publishes them
  asm volatile("s_barrier" ::: "memory");
  f32x4 s[2][RB];
  pl.scores(pl.stage(0), koff, qr, s);

  uint32_t sp = 0;  // byte offset of pair p's stage buffer
  for (int p = 0; p < npairs; ++p) {
    asm volatile("" : "+s"(sp));  // one opaque scalar (see stage_off)
    pl.base_q = p;
    pl.base_off = sp;
    // Own copies of pair p + kA complete: at most the later pairs' copies
    // (p + kA + 1 .. p + S - 2) stay outstanding.
    wait_stages<SG::kLoads, S - 2 - kA>(max(0, min(S - 2 - kA, npairs - 1 - kA - p)));
    // The barrier makes pair p + kA complete for all waves, publishes the
    // rotation of pair p + 1, and frees buffer (p - 1) % S (its V was read
    // at iteration p - 1, its K at p - 2).  A bare s_barrier (compiler
    // memory clobber only): a fenced __syncthreads would also drain the
    // copies of the later pairs still in flight.
    asm volatile("s_barrier" ::: "memory");
    // headers for the next iteration (written at least two barriers ago)
    const u32x4 hv_next = pl.read_hdr(p + 1);
    u32x2 dv_next = {0u, 0u};
    if constexpr (P::kRot) dv_next = pl.read_deltas(p + 3);
    // the next pair's document offset (the per-document query rotation)
    int dq_next = dq_cur;
    if constexpr (P::kQRot) dq_next = (p + 1 < npairs) ? uniform((int)pl.read_deltas(p + 1)[0]) : dq_cur;
    // Rotation of pair p + 2 in two halves: its LDS reads now, its
    // arithmetic and write-back (with the next copies) in the other half of
    // the iteration from this pair's softmax and products.
    typename P::RotWork rot;
#pragma unroll
    for (int k = 0; k < P::kRI; ++k) rot.it[k].on = false;
    if (p + 2 < npairs) rot = pl.rot_load(p + 2, dr);
    // The two waves of a SIMD take the iteration's halves in opposite
    // orders: waves 0..3 the softmax and products first, then the rotation
    // and copies; waves 4..7 the other way round.  Each wave's matrix-heavy
    // half then overlaps the other's vector and LDS half.
    const bool copy_first = wave >= NW / 2;
    if (copy_first) {
      pl.rot_store(rot);  // rotation of pair p + 2
      if (p + S - 1 < npairs) pl.issue(p + S - 1, wi);
    }
    if (has_rows) {
      const unsigned char* st = pl.stage(p);

      // V^T operand of channel block n: the 8 tokens this lane's scores hold
      F8 vv[NV];
#pragma unroll
      for (int n = 0; n < NV; ++n) vv[n] = *reinterpret_cast<const F8*>(st + voff + n * 512);

      // Masking only where a slot can be invalid: partial or dropped tiles,
      // causal private tiles, ALiBi bias (wave-uniform test on the words).
      const bool full = (hc[3] & kHdrFull) != 0u;
      if (!full) {
        const bool hi = g >= 2;
        const uint32_t msk = hi ? (hc[0] >> 16) : (hc[0] & 0xFFFFu);
        const int off = (int)(hi ? hc[2] : hc[1]);
        const bool pv = (hc[3] & (hi ? kHdrPriv1 : kHdrPriv0)) != 0u;
        // fill bits of this lane's eight tokens 8 (g % 2) + t (t = the slot in
        // its score and V fragments)
        const uint32_t m8 = (msk >> (8 * (g & 1))) & 0xFFu;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int tok = 8 * (g & 1) + 4 * h + j;
            const bool filled = (m8 >> (4 * h + j)) & 1u;
            const int kpos = off + tok;
#pragma unroll
            for (int b = 0; b < RB; ++b) {
              const bool ok = filled && (!pv || kpos <= qp[b]);
              float v = s[h][b][j];
              if (KIND == kAlibi) v = fmaf(slope_raw[b], (float)(kpos - qp[b]), v);
              s[h][b][j] = ok ? v : -INFINITY;
            }
          }
        }
        // Empty slots hold unwritten pool bytes: zero their V (their weight is
        // 0, but 0 x NaN is not).  Every channel block of the lane has the same
        // eight slots, so one AND mask per dword (two bf16 slots) covers all.
        u32x4 dm;
#pragma unroll
        for (int d = 0; d < 4; ++d)
          dm[d] = (((m8 >> (2 * d)) & 1u) ? 0x0000FFFFu : 0u) | (((m8 >> (2 * d + 1)) & 1u) ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int n = 0; n < NV; ++n) vv[n] = __builtin_bit_cast(F8, __builtin_bit_cast(u32x4, vv[n]) & dm);
      }

      // Lazy rescale: the reference max m_run only moves (and acc, l are
      // rescaled) when some row's score exceeds it by more than 2^SLACK, so
      // every weight stays <= 2^SLACK; exact in real arithmetic, and the combine
      // uses the same reference.  Checked per lane on raw scores (scale > 0).
      float mx[RB];
      bool grow = false;
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        float m = fmaxf(fmaxf(s[0][b][0], s[0][b][1]), fmaxf(s[0][b][2], s[0][b][3]));
        m = fmaxf(m, fmaxf(fmaxf(s[1][b][0], s[1][b][1]), fmaxf(s[1][b][2], s[1][b][3])));
        mx[b] = m;
        grow = grow || (m > thr[b]);
      }
      if (__any(grow)) {
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const float m_new = fmaxf(m_run[b], xor_max16_32(mx[b]) * sl);
          const float alpha = (m_run[b] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[b] - m_new);
#pragma unroll
          for (int n = 0; n < NV; ++n) acc[b][n] *= alpha;
          lsum[b] *= alpha;
          m_run[b] = m_new;
          const bool none = m_new == -INFINITY;
          negm[b] = none ? 0.f : -m_new;
          thr[b] = none ? -INFINITY : (m_new + (float)LAZY_RESCALE_SLACK) / sl;
        }
      }

      if constexpr (P::kQRot) {
        // a new document from the next pair on: the query rotated for it
        // before the exponentials, so they, the next pair's scores and the
        // P V products stay one straight-line block (the next pair's stage
        // and cos/sin row landed before this iteration's barrier)
        if (dq_next != dq_cur) {
          if (dq_next == 0) {
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
              for (int c = 0; c < NC; ++c) qr[b][c] = *reinterpret_cast<const F8*>(pl.lds + pl.q_slot(b, c));
          } else {
            pl.rotate_q(p + 1, qr);
          }
          dq_cur = dq_next;
        }
      }
      // weights p = 2^(s * scale_log2 - m_run), row sums and P V on the
      // MFMAs, with the next pair's scores in the same straight-line block
      // (their products overlap this pair's exponentials); past the last pair
      // they are computed from a stale buffer and never used
      F8 pf[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 4; ++j) pf[b][4 * h + j] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[h][b][j], sl, negm[b]));
      pl.scores(pl.stage(p + 1), koff, qr, s);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        lsum[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[b], lsum[b], 0, 0, 0);
#pragma unroll
        for (int n = 0; n < NV; ++n) acc[b][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv[n], pf[b], acc[b][n], 0, 0, 0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
    if (!copy_first) {
      pl.rot_store(rot);  // rotation of pair p + 2 (its LDS reads were issued before the products)
      if (p + S - 1 < npairs) pl.issue(p + S - 1, wi);
    }
    wi = pl.load_words(p + S);
#pragma unroll
    for (int k = 0; k < 4; ++k) hc[k] = (uint32_t)uniform((int)hv_next[k]);
    dr[0] = uniform((int)dv_next[0]);
    dr[1] = uniform((int)dv_next[1]);
    sp = pl.stage_off(p + 1);
  }
}

template <int DH, int KIND, bool DEFER, int RB, int NW, bool QROT>
__global__ __launch_bounds__(64 * NW, 1) void prefill_lds_kernel(AttnArgs a, int row_tiles, int num_wgs) {
  using P = LdsPrefill<DH, KIND, DEFER, RB, NW, 10, false, QROT>;
  using F8 = typename P::F8;
  using F4 = typename P::F4;
  constexpr int NC = P::NC;
  constexpr int NV = P::NV;
  extern __shared__ __align__(16) unsigned char lds_buf[];

  // ids through the intrinsics (no library call: a call's results would
  // not be known to be wave-uniform)
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  int req, kvh, split, row_tile;
  xcd_unit(__builtin_amdgcn_workgroup_id_x(), num_wgs, a.num_splits, a.hkv, row_tiles, req, kvh, split, row_tile);

  const int q0 = a.q_start[req];
  int nq = a.q_start[req + 1] - q0;
  nq = min(nq, a.max_q_len);
  nq = max(0, min(nq, a.rows_bound / a.hq - q0));
  const int nrows = nq * a.group;
  const int t0 = a.tile_start[req];
  const int nt = a.tile_start[req + 1] - t0;
  int sb, se;
  // workgroup-uniform exits only (barriers follow)
  if (row_tile * NW * RB * 16 >= nrows) return;
  if (!split_range(nt, a.chunk, a.num_splits, split, sb, se)) return;
  const int npairs = (se - sb + 1) >> 1;
  const int rb0 = (row_tile * NW + wave) * RB;
  const bool has_rows = rb0 * 16 < nrows;  // wave-uniform: waves without rows still copy and rotate
  const int qpos0 = a.q_pos[req];

  P pl{a, lds_buf, tid, lane, wave, kvh, sb, se, a.ctx_tiles[req], npairs, (const_words)(a.tiles + t0), {}};
  pl.init_copies();

  // Query rows at their global positions: row rho of the request is
  // (token rho / G, head kvh*G + rho % G); rows past the request's last are
  // zero (computed, never stored).
  int qp[RB];
  float slope_raw[RB];
  F8 qr[RB][NC];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int rho = (rb0 + b) * 16 + r;
    const bool ok = rho < nrows;
    const int qi = ok ? rho / a.group : 0;
    const int head = kvh * a.group + (ok ? rho % a.group : 0);
    qp[b] = qpos0 + qi;
    // ALiBi in the raw-score domain: bias / softmax scale
    slope_raw[b] = (KIND == kAlibi) ? a.slopes[head] * kLog2e / a.scale_log2 : 0.f;
    const bf16* qrow = reinterpret_cast<const bf16*>(a.q) + ((int64_t)(q0 + qi) * a.hq + head) * DH;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const F8 v = *reinterpret_cast<const F8*>(qrow + 32 * c + 8 * g);
      qr[b][c] = ok ? v : F8{};
    }
  }

  f32x4 acc[RB][NV];
  f32x4 lsum[RB];
  float m_run[RB];
  lds_attend<DH, KIND, DEFER, RB, NW, 10, false, QROT>(pl, qr, qp, slope_raw, has_rows, acc, lsum, m_run);
  if (!has_rows) return;

  // O[row r][16n + 4g + j] = acc[b][n][j]: normalised output (one split) or an
  // unnormalised (m, l, acc) partial for the combine.
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int rho = (rb0 + b) * 16 + r;
    if (rho >= nrows) continue;
    const int orow = (q0 + rho / a.group) * a.hq + kvh * a.group + rho % a.group;
    const float l_tot = lsum[b][0];
    if (a.num_splits == 1) {
      const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
      bf16* o = reinterpret_cast<bf16*>(a.out) + (int64_t)orow * DH + 4 * g;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        F4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = (bf16)(acc[b][n][j] * inv);
        *reinterpret_cast<F4*>(o + 16 * n) = w;
      }
    } else {
      const int64_t prow = (int64_t)split * a.rows_bound + orow;
      float* po = a.part_o + prow * DH + 4 * g;
#pragma unroll
      for (int n = 0; n < NV; ++n) *reinterpret_cast<f32x4*>(po + 16 * n) = acc[b][n];
      if (g == 0) {
        a.part_ml[prow * 2 + 0] = m_run[b];
        a.part_ml[prow * 2 + 1] = l_tot;
      }
    }
  }
}

// The document pass of the document-major decode on the same ring: one
// workgroup per (work item, KV head), a work item being up to NW x RB x 16
// rows (reads of one shared document x the query group) against one chunk of
// the document's tiles.  The tiles are copied once per workgroup for all
// those rows; each row's query is rotated by -Delta of its read on the way
// into registers (the single relative rotation, LazyAttention notes,
// "Key designs": decode rotates the query) and the keys stay at their local
// positions, so the ring runs without its K rotation.  Every row ends as an
// (m, l, acc) partial in its read's slot (one per chunk), which the decode
// combine merges with the request's other partials.  Grid (KV head, work
// item): with eight KV heads a head is one XCD, and a document's row tiles
// are adjacent items there, so the second one finds the tiles in L2.  The
// accumulators go out in bf16 (DocPassArgs::doc_o), m and l in fp32.
template <int DH, int KIND, int RB, int NW, int MAXS, int WPE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE))) void docpass_lds_kernel(
    AttnArgs a, DocPassArgs d) {
  using P = LdsPrefill<DH, KIND, false, RB, NW, MAXS, true>;
  using F8 = typename P::F8;
  constexpr int NC = P::NC;
  constexpr int NV = P::NV;
  extern __shared__ __align__(16) unsigned char lds_buf[];

  const int tid = __builtin_amdgcn_workitem_id_x();
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int kvh = __builtin_amdgcn_workgroup_id_x();
  const int item = __builtin_amdgcn_workgroup_id_y();
  const int doc = d.work[4 * item];
  const int b0 = d.work[4 * item + 1];
  const int chunk = d.work[4 * item + 2];
  const int ct = d.work[4 * item + 3];
  const int dt0 = d.doc_tile_start[doc];
  const int nt_doc = d.doc_tile_start[doc + 1] - dt0;
  const int tb = min(nt_doc, chunk * ct);
  const int nt = min(nt_doc - tb, ct);
  const int read0 = d.read_start[doc];
  const int nrows = (d.read_start[doc + 1] - read0) * a.group;
  // workgroup-uniform exits only (barriers follow)
  if (b0 * 16 >= nrows || nt <= 0) return;
  const int npairs = (nt + 1) >> 1;
  const int rb0 = b0 + wave * RB;
  const bool has_rows = rb0 * 16 < nrows;

  // every tile of the chunk is a context tile at its local position
  P pl{a, lds_buf, tid, lane, wave, kvh, 0, nt, nt, npairs, (const_words)(d.doc_tiles + dt0 + tb), {}};
  pl.init_copies();

  // Row rho = (read rho / G, head kvh*G + rho % G): that request's query
  // rotated by -Delta; ALiBi measures the distance from q_pos - Delta, the
  // keys sitting at Delta + their local positions.  A Delta the table cannot
  // serve is never looked up: its rows' partials are stored as NaN bit
  // patterns (this file is built without NaN semantics, so no NaN value is
  // ever computed here).
  int qp[RB], delta[RB];
  float slope_raw[RB];
  int64_t prow[RB];
  bool bad[RB];
  const bf16* qptr[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int rho = (rb0 + b) * 16 + r;
    const int rr = rho < nrows ? rho : 0;
    int req, slot, dl;
    unpack_read(d.reads[read0 + rr / a.group], req, slot, dl);
    const int head = kvh * a.group + rr % a.group;
    qptr[b] = reinterpret_cast<const bf16*>(a.q) + ((int64_t)req * a.hq + head) * DH;
    qp[b] = a.q_pos[req] - dl;
    slope_raw[b] = (KIND == kAlibi) ? a.slopes[head] * kLog2e / a.scale_log2 : 0.f;
    prow[b] = (int64_t)(d.slot_base + slot + chunk) * a.rows_bound + ((int64_t)req * a.hq + head);
    bad[b] = KIND != kAlibi && a.cos_sin != nullptr && (dl < 0 || dl >= a.max_pos);
    delta[b] = (KIND == kAlibi || bad[b]) ? 0 : dl;
  }
  F8 qr[RB][NC];
  const int active = has_rows ? min(RB, (nrows - rb0 * 16 + 15) / 16) : 0;
  rotate_query_rows<bf16, DH, KIND, RB>(qr, qptr, a, delta, g, active);

  f32x4 acc[RB][NV];
  f32x4 lsum[RB];
  float m_run[RB];
  lds_attend<DH, KIND, false, RB, NW, MAXS, true, false>(pl, qr, qp, slope_raw, has_rows, acc, lsum, m_run);
  if (!has_rows) return;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    if ((rb0 + b) * 16 + r >= nrows) continue;
    // the accumulator in bf16 in the reads' own rows; (m, l) in fp32 in the
    // slot's part_ml row
    bf16* po = reinterpret_cast<bf16*>(d.doc_o) + (prow[b] - (int64_t)d.slot_base * a.rows_bound) * DH + 4 * g;
    if (bad[b]) {
      constexpr uint32_t kQNaN = 0x7FC00000u, kQNaN2 = 0x7FC07FC0u;
      const u32x2 nan_o = {kQNaN2, kQNaN2};
#pragma unroll
      for (int n = 0; n < NV; ++n) *reinterpret_cast<u32x2*>(po + 16 * n) = nan_o;
      if (g == 0) {
        const u32x2 nan2 = {kQNaN, kQNaN};
        *reinterpret_cast<u32x2*>(a.part_ml + prow[b] * 2) = nan2;
      }
      continue;
    }
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      bf16x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = (bf16)acc[b][n][j];
      *reinterpret_cast<bf16x4*>(po + 16 * n) = w;
    }
    if (g == 0) {
      a.part_ml[prow[b] * 2 + 0] = m_run[b];
      a.part_ml[prow[b] * 2 + 1] = lsum[b][0];
    }
  }
}

namespace {

// The ring needs more than the default 64 KiB of dynamic LDS: the attribute
// is set once per device and kernel (a second setting is harmless, so racing
// threads need no lock).
template <const void* (*KERNEL)()>
hipError_t ensure_lds_attr(size_t lds) {
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0ull;
  if (bit == 0 || !(attr_set.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(KERNEL(), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_release);
  }
  return hipSuccess;
}

template <int DH, int KIND, bool DEFER, int RB, int NW, bool QROT>
const void* prefill_kernel_ptr() {
  return reinterpret_cast<const void*>(&prefill_lds_kernel<DH, KIND, DEFER, RB, NW, QROT>);
}

template <int DH, int KIND, int RB, int NW, int MAXS, int WPE>
const void* docpass_kernel_ptr() {
  return reinterpret_cast<const void*>(&docpass_lds_kernel<DH, KIND, RB, NW, MAXS, WPE>);
}

template <int DH, int KIND, bool DEFER, int RB, bool QROT>
hipError_t launch_rb(const AttnArgs& a, int row_tiles, int splits, int num_reqs, int hkv, hipStream_t st) {
  constexpr int NW = kPrefillWaves;
  using SG = typename LdsPrefill<DH, KIND, DEFER, RB, NW, 10, false, QROT>::SG;
  const size_t lds = (size_t)SG::kLdsTotal;
  hipError_t e = ensure_lds_attr<prefill_kernel_ptr<DH, KIND, DEFER, RB, NW, QROT>>(lds);
  if (e != hipSuccess) return e;
  const int num_wgs = row_tiles * splits * hkv * num_reqs;  // 1-D: the kernel maps ids to units
  hipLaunchKernelGGL((prefill_lds_kernel<DH, KIND, DEFER, RB, NW, QROT>), dim3((unsigned)num_wgs), dim3(64 * NW), lds,
                     st, a, row_tiles, num_wgs);
  return hipGetLastError();
}

// rows per workgroup = 16 x rb x 4 (the host plan's row tile) = NW waves x (4 rb / NW) blocks
template <int DH, int KIND, bool DEFER, bool QROT>
hipError_t launch_kind(const AttnArgs& a, int rb, int row_tiles, int splits, int num_reqs, int hkv, hipStream_t st) {
  constexpr int NW = kPrefillWaves;
  static_assert(NW == 4 || NW == 8, "waves per workgroup");
  return rb == 4 ? launch_rb<DH, KIND, DEFER, 16 / NW, QROT>(a, row_tiles, splits, num_reqs, hkv, st)
                 : launch_rb<DH, KIND, DEFER, 8 / NW, QROT>(a, row_tiles, splits, num_reqs, hkv, st);
}

// qrot: the tile pairs keep to one document (LAZY_FLAG_DOC_PAIRS): the query
// is rotated per document instead of K per pair
template <int DH>
hipError_t launch_dh(const AttnArgs& a, int kind, bool defer, bool qrot, int rb, int row_tiles, int splits,
                     int num_reqs, int hkv, hipStream_t st) {
  switch (kind) {
    case kHalf:
      if (!defer) return launch_kind<DH, kHalf, false, false>(a, rb, row_tiles, splits, num_reqs, hkv, st);
      return qrot ? launch_kind<DH, kHalf, true, true>(a, rb, row_tiles, splits, num_reqs, hkv, st)
                  : launch_kind<DH, kHalf, true, false>(a, rb, row_tiles, splits, num_reqs, hkv, st);
    case kInter:
      if (!defer) return launch_kind<DH, kInter, false, false>(a, rb, row_tiles, splits, num_reqs, hkv, st);
      return qrot ? launch_kind<DH, kInter, true, true>(a, rb, row_tiles, splits, num_reqs, hkv, st)
                  : launch_kind<DH, kInter, true, false>(a, rb, row_tiles, splits, num_reqs, hkv, st);
    default:
      return launch_kind<DH, kAlibi, false, false>(a, rb, row_tiles, splits, num_reqs, hkv, st);
  }
}

}  // namespace

namespace {

template <int DH, int KIND>
hipError_t launch_docpass_dh(const AttnArgs& a, const DocPassArgs& d, int num_work, int hkv, hipStream_t st) {
  constexpr int NW = kDocPassLdsWaves;
  constexpr int RB = kDocPassLdsRb;
  constexpr int MAXS = LAZY_DOCPASS_STAGES;
  constexpr int WPE = LAZY_DOCPASS_LDS_WPE;
  using SG = StageGeom<DH, false, NW, MAXS>;
  const size_t lds = (size_t)SG::kLdsTotal;
  hipError_t e = ensure_lds_attr<docpass_kernel_ptr<DH, KIND, RB, NW, MAXS, WPE>>(lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((docpass_lds_kernel<DH, KIND, RB, NW, MAXS, WPE>), dim3((unsigned)hkv, (unsigned)num_work),
                     dim3(64 * NW), lds, st, a, d);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_docpass_kind(const AttnArgs& a, const DocPassArgs& d, int kind, int num_work, int hkv,
                               hipStream_t st) {
  switch (kind) {
    case kHalf:
      return launch_docpass_dh<DH, kHalf>(a, d, num_work, hkv, st);
    case kInter:
      return launch_docpass_dh<DH, kInter>(a, d, num_work, hkv, st);
    default:
      return launch_docpass_dh<DH, kAlibi>(a, d, num_work, hkv, st);
  }
}

}  // namespace

hipError_t launch_docpass_lds(const AttnArgs& a, const DocPassArgs& d, int kind, int head_dim, int num_work, int hkv,
                              hipStream_t st) {
  if (num_work <= 0) return hipSuccess;
  if (head_dim == 128) return launch_docpass_kind<128>(a, d, kind, num_work, hkv, st);
  if (head_dim == 64) return launch_docpass_kind<64>(a, d, kind, num_work, hkv, st);
  return hipErrorNotSupported;
}

hipError_t launch_prefill_lds(const AttnArgs& a, int kind, bool defer, int head_dim, int rb, int row_tiles,
                              int splits, int num_reqs, int hkv, hipStream_t st) {
  const bool qrot = a.doc_pairs != 0;
  if (rb != 2 && rb != 4) return hipErrorNotSupported;
  if (kind != kAlibi && defer && a.cos_sin == nullptr) return hipErrorNotSupported;  // rows come from the table
  if (head_dim == 128) return launch_dh<128>(a, kind, defer, qrot, rb, row_tiles, splits, num_reqs, hkv, st);
  if (head_dim == 64) return launch_dh<64>(a, kind, defer, qrot, rb, row_tiles, splits, num_reqs, hkv, st);
  return hipErrorNotSupported;
}

}  // namespace lazy
