// Shared device pieces of the attention kernels: arguments, tuning knobs,
// query rotation, the per-wave attention state (scores, online softmax, PV)
// and split-K bookkeeping.  Included by the kernel translation units.
#pragma once

#include <math.h>

#include <algorithm>

#include "lazy_device.hpp"
#include "lazy_host.hpp"

// Compile-time tuning knobs (defaults are the measured best on MI355X).
//
// Decode loop shape: 1 = software-pipelined (next pair's K/V in flight while
// the current pair is consumed; doubles fragment registers, one wave per
// SIMD), 0 = load-then-consume per pair with the next tile words prefetched.
#ifndef LAZY_DECODE_PIPELINE
#define LAZY_DECODE_PIPELINE 0
#endif
// Decode split heuristic: about this many waves (one per split and (request,
// KV head)) per launch.  Requests of near-uniform length: one resident round
// on 256 CUs at two waves per SIMD (more splits only add partials and tail).
// Uneven lengths: four rounds at three waves per SIMD (the launch picks the
// three-wave build for them), so the dispatcher can balance waves that
// progress at different speeds (measured on MI355X: 64 x 32K uniform batch
// best at 2048; 48 x 8K-66K batch with shared documents 812 us at 12288
// waves and three per SIMD, 852 us at 8192 and two, 886 us at 12288 and two).
#ifndef LAZY_DECODE_WAVE_TARGET
#define LAZY_DECODE_WAVE_TARGET 2048
#endif
#ifndef LAZY_DECODE_WAVE_TARGET_UNEVEN
#define LAZY_DECODE_WAVE_TARGET_UNEVEN 12288
#endif
// Decode: fewest tiles per split.
#ifndef LAZY_DECODE_MIN_CHUNK
#define LAZY_DECODE_MIN_CHUNK 16
#endif
// Document pass: waves per SIMD the build is register-capped for (2 fits its
// 200 registers without spills; the uncapped build drifts past 256 and runs
// one wave per SIMD, 0.47 vs 0.37 ms on the mixed step's decode; 3 spills).
#ifndef LAZY_DOCPASS_WPE
#define LAZY_DOCPASS_WPE 2
#endif
// Prefill split heuristic: about this many workgroups per launch.
#ifndef LAZY_PREFILL_WG_TARGET
#define LAZY_PREFILL_WG_TARGET 256
#endif
// 1: wave index through readfirstlane (tile words via the scalar cache);
// 0: plain thread index (tile words via vector loads), measured faster.
#ifndef LAZY_UNIFORM_WAVE
#define LAZY_UNIFORM_WAVE 0
#endif
// Decode row blocks per wave: 1 = the smallest count of 16-row blocks that
// holds a KV head's query group (3 and 5 included), 0 = powers of two only.
#ifndef LAZY_DECODE_RB_EXACT
#define LAZY_DECODE_RB_EXACT 1
#endif
// Waves per SIMD the dh-64 decode builds with three or more row blocks are
// register-capped for (1 = no cap).
#ifndef LAZY_DECODE_MANY_ROWS_WPE
#define LAZY_DECODE_MANY_ROWS_WPE 2
#endif
// Online softmax: rescale only when a row max grows by more than 2^SLACK.
#ifndef LAZY_RESCALE_SLACK
#define LAZY_RESCALE_SLACK 8
#endif

namespace lazy {

struct AttnArgs {
  const void* k_cache;
  const void* v_cache;
  int64_t num_blocks;
  const uint64_t* tiles;
  const int32_t* tile_start;
  const int32_t* ctx_tiles;
  const void* q;
  const int32_t* q_start;  // prefill: row range per request; decode: unused (row r = request r)
  const int32_t* q_pos;    // prefill: position of the first query row; decode: query position
  const float* cos_sin;    // [max_pos][DH] or NULL (on-the-fly from inv_freq)
  const double* inv_freq;
  int32_t max_pos;
  const float* slopes;
  float scale_log2;  // softmax_scale * log2(e)
  void* out;
  float* part_o;  // [splits][rows_bound][DH]
  float* part_ml;  // [splits][rows_bound][2]
  int32_t num_splits;  // grid extent along splits (largest per-request split count)
  int32_t chunk;       // tiles per split (even); request r uses ceil(nt_r / chunk) splits
  int32_t hq, hkv, group;
  int32_t rows_bound;  // partial row stride: (max query rows) * hq
  int32_t max_q_len;   // prefill: rows per request covered by the grid
  int32_t force_partials;  // write (m, l, acc) partials even with one split (a later combine merges more)
  int32_t doc_pairs;       // prefill: no tile pair spans two documents (LAZY_FLAG_DOC_PAIRS)
};

// The document-major pass of a decode batch: each shared document's tiles
// (cached at local positions; tile offset = local position of slot 0) and
// the reads of it, one per (request, placement).  Read word: request
// [63:48] | partial slot of that request [47:32] | Delta [31:0].
struct DocPassArgs {
  const uint64_t* doc_tiles;
  const int32_t* doc_tile_start;  // [num_docs + 1]
  const int32_t* read_start;      // [num_docs + 1]
  const uint64_t* reads;          // [num_reads]
  const int32_t* work;            // [num_work][4]: (doc, first 16-row block, chunk, tiles per chunk)
  int32_t slot_base;              // partial slots of a request's reads start at slot_base (in part_ml)
  // the reads' accumulators, [max_req_reads][rows_bound][dh] in the call's
  // dtype (fp32: the rows right after the split slots' part_o rows)
  void* doc_o;
};

__device__ __forceinline__ void unpack_read(uint64_t w, int& req, int& slot, int& delta) {
  req = (int)(w >> 48);
  slot = (int)((w >> 32) & 0xFFFFull);
  delta = (int)(w & 0xFFFFFFFFull);
}

enum { kHalf = LAZY_ROPE_HALF, kInter = LAZY_ROPE_INTERLEAVED, kAlibi = LAZY_ALIBI };

// cos/sin of Delta * theta_k for the rotation pairs of one chunk a lane owns.
// Half-split: chunk c < DH/64 holds pairs k = 32c + 8g + t (t < 8), the
// partner channels sitting in chunk c + DH/64 of the same lane.
// Interleaved: chunk c < DH/32 holds pairs k = 16c + 4g + u (u < 4), channels
// (2k, 2k+1) adjacent inside the lane's eight values.
template <int DH, int KIND>
__device__ __forceinline__ void chunk_coefs(const AttnArgs& a, int delta, int g, int c, float (&cs)[8],
                                            float (&sn)[8]) {
  constexpr int N = (KIND == kHalf) ? 8 : 4;
  const int k0 = (KIND == kHalf) ? 32 * c + 8 * g : 16 * c + 4 * g;
  if (a.cos_sin != nullptr) {
    const float* row = a.cos_sin + (int64_t)delta * DH + k0;
#pragma unroll
    for (int h = 0; h < N / 4; ++h) {
      const f32x4 c4 = *reinterpret_cast<const f32x4*>(row + 4 * h);
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(row + DH / 2 + 4 * h);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        cs[4 * h + t] = c4[t];
        sn[4 * h + t] = s4[t];
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < N; ++t) sincos_reduced(delta, a.inv_freq[k0 + t], &sn[t], &cs[t]);  // no table reads
  }
}

// q' = R_{-delta} q for the RB row blocks of this wave: one chunk of rotation
// pairs at a time (lane-local pairs), so only that chunk's coefficients and
// raw values are live.
template <typename T, int DH, int KIND, int RB>
__device__ __forceinline__ void rotate_query(typename Elem<T>::Frag8 (&qr)[RB][DH / 32], const T* const (&qptr)[RB],
                                             const AttnArgs& a, int delta, int g, int active_blocks) {
  using E = Elem<T>;
  using F8 = typename E::Frag8;
  constexpr int NC = DH / 32;
  // Row blocks past the wave's last row keep a zero query: their products
  // are computed (so no load is ever predicated) and discarded.
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    if (b >= active_blocks) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int t = 0; t < 8; ++t) qr[b][c][t] = E::from_f(0.f);
    }
  }
  if (KIND == kAlibi || delta == 0) {
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if (b >= active_blocks) continue;
#pragma unroll
      for (int c = 0; c < NC; ++c) qr[b][c] = load8<T>(qptr[b] + 32 * c + 8 * g);
    }
    return;
  }
  if (KIND == kHalf) {
#pragma unroll
    for (int c = 0; c < NC / 2; ++c) {
      float cs[8], sn[8];
      chunk_coefs<DH, KIND>(a, delta, g, c, cs, sn);
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        if (b >= active_blocks) continue;
        const F8 lo = load8<T>(qptr[b] + 32 * c + 8 * g);
        const F8 hi = load8<T>(qptr[b] + 32 * (c + NC / 2) + 8 * g);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float x1 = E::to_f(lo[t]), x2 = E::to_f(hi[t]);
          qr[b][c][t] = E::from_f(x1 * cs[t] + x2 * sn[t]);  // rotation by -delta
          qr[b][c + NC / 2][t] = E::from_f(x2 * cs[t] - x1 * sn[t]);
        }
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float cs[8], sn[8];
      chunk_coefs<DH, KIND>(a, delta, g, c, cs, sn);
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        if (b >= active_blocks) continue;
        const F8 x = load8<T>(qptr[b] + 32 * c + 8 * g);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float x1 = E::to_f(x[2 * u]), x2 = E::to_f(x[2 * u + 1]);
          qr[b][c][2 * u] = E::from_f(x1 * cs[u] + x2 * sn[u]);
          qr[b][c][2 * u + 1] = E::from_f(x2 * cs[u] - x1 * sn[u]);
        }
      }
    }
  }
}

// q' = R_{-delta_b} q for each row block b with a delta of its own per lane
// row (the document-major pass: every row is one request's read of the same
// document at that request's offset).  Same pairing as rotate_query.
template <typename T, int DH, int KIND, int RB>
__device__ __forceinline__ void rotate_query_rows(typename Elem<T>::Frag8 (&qr)[RB][DH / 32],
                                                  const T* const (&qptr)[RB], const AttnArgs& a,
                                                  const int (&delta)[RB], int g, int active_blocks) {
  using E = Elem<T>;
  constexpr int NC = DH / 32;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    if (b >= active_blocks) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int t = 0; t < 8; ++t) qr[b][c][t] = E::from_f(0.f);
      continue;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) qr[b][c] = load8<T>(qptr[b] + 32 * c + 8 * g);
    if (KIND == kAlibi) continue;
    if (KIND == kHalf) {
#pragma unroll
      for (int c = 0; c < NC / 2; ++c) {
        float cs[8], sn[8];
        chunk_coefs<DH, KIND>(a, delta[b], g, c, cs, sn);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float x1 = E::to_f(qr[b][c][t]), x2 = E::to_f(qr[b][c + NC / 2][t]);
          qr[b][c][t] = E::from_f(x1 * cs[t] + x2 * sn[t]);
          qr[b][c + NC / 2][t] = E::from_f(x2 * cs[t] - x1 * sn[t]);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float cs[8], sn[8];
        chunk_coefs<DH, KIND>(a, delta[b], g, c, cs, sn);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float x1 = E::to_f(qr[b][c][2 * u]), x2 = E::to_f(qr[b][c][2 * u + 1]);
          qr[b][c][2 * u] = E::from_f(x1 * cs[u] + x2 * sn[u]);
          qr[b][c][2 * u + 1] = E::from_f(x2 * cs[u] - x1 * sn[u]);
        }
      }
    }
  }
}

// Per-wave attention state: RB blocks of 16 query rows of one (request, KV
// head) against a stream of tile pairs.  Shared by the prefill and decode
// kernels.  Query row rho of a request is (token rho / G, head kvh*G + rho % G).
template <typename T, int DH, int KIND, bool DEFER, bool PREFILL, int RB, int NQ_ = -1>
struct WaveAttn {
  using E = Elem<T>;
  using F8 = typename E::Frag8;
  using F4 = typename E::Frag4;
  static constexpr int NC = DH / 32;  // contraction chunks of QK^T
  static constexpr int NV = DH / 16;  // 16-channel blocks of the output
  static constexpr bool kRot = (KIND != kAlibi) && DEFER;
  // Rotated query per tile slot of a pair (x = 0: even tile, 1: odd tile), so
  // a pair that straddles a document boundary needs no re-rotation between
  // its two QK^T products; a document costs at most two rotations.
  static constexpr int NQ = (NQ_ > 0) ? NQ_ : (kRot ? 2 : 1);

  struct Pair {
    TileMeta mt[2];
    int delta[2];
    bool priv[2];
  };
  struct Frags {
    F8 k[2][NC];
    F4 v[2][NV];
  };

  const AttnArgs& a;
  int r, g, kvh, t0, nctx, active_blocks;
  const T* qptr[RB];
  int qp[RB];
  int orow[RB];
  bool rvalid[RB];
  float slope2[RB];
  F8 qr[NQ][RB][NC];
  int pslot[RB];  // partial slot of each row (-1: the wave's split)
  int cur_delta[2];
  f32x4 acc[RB][NV];
  float m_run[RB], l_run[RB];

  __device__ __forceinline__ WaveAttn(const AttnArgs& a_, int lane, int kvh_, int req, int q0, int nrows, int rb0,
                                      int qpos0)
      : a(a_) {
    r = lane & 15;
    g = lane >> 4;
    kvh = kvh_;
    t0 = a.tile_start[req];
    nctx = a.ctx_tiles[req];
    active_blocks = min(RB, (nrows - rb0 * 16 + 15) / 16);
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int rho = (rb0 + b) * 16 + r;
      rvalid[b] = rho < nrows;
      const int rr = rvalid[b] ? rho : 0;
      const int qi = rr / a.group;
      const int head = kvh * a.group + rr % a.group;
      qptr[b] = reinterpret_cast<const T*>(a.q) + ((int64_t)(q0 + qi) * a.hq + head) * DH;
      qp[b] = qpos0 + qi;
      orow[b] = (q0 + qi) * a.hq + head;
      slope2[b] = (KIND == kAlibi) ? a.slopes[head] * kLog2e : 0.f;
    }
    rotate_query<T, DH, KIND, RB>(qr[0], qptr, a, 0, g, active_blocks);
    if (NQ > 1) {
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int c = 0; c < NC; ++c) qr[NQ - 1][b][c] = qr[0][b][c];
    }
    cur_delta[0] = cur_delta[1] = 0;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      pslot[b] = -1;
      m_run[b] = -INFINITY;
      l_run[b] = 0.f;
#pragma unroll
      for (int n = 0; n < NV; ++n) acc[b][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // Document-major pass: the wave's rows are reads of one shared document,
  // row rho = (read rho / G, head kvh * G + rho % G); each read's query is
  // rotated once by -Delta of that read, the document's keys stay at their
  // local positions, and every row's partial goes to its request's slot.
  struct DocRows {};
  __device__ __forceinline__ WaveAttn(const AttnArgs& a_, const DocPassArgs& d, int lane, int kvh_, int doc, int nrows,
                                      int rb0, int chunk, int chunk_tiles, DocRows)
      : a(a_) {
    r = lane & 15;
    g = lane >> 4;
    kvh = kvh_;
    // this wave's chunk of the document's tiles (every tile a context tile);
    // chunk c of a read lands in the read's slot + c
    const int dt0 = d.doc_tile_start[doc];
    const int nt_doc = d.doc_tile_start[doc + 1] - dt0;
    const int tb = min(nt_doc, chunk * chunk_tiles);
    t0 = dt0 + tb;
    nctx = min(nt_doc - tb, chunk_tiles);
    active_blocks = min(RB, (nrows - rb0 * 16 + 15) / 16);
    const int read0 = d.read_start[doc];
    int delta[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int rho = (rb0 + b) * 16 + r;
      rvalid[b] = rho < nrows;
      const int rr = rvalid[b] ? rho : 0;
      int req, slot;
      unpack_read(d.reads[read0 + rr / a.group], req, slot, delta[b]);
      const int head = kvh * a.group + rr % a.group;
      qptr[b] = reinterpret_cast<const T*>(a.q) + ((int64_t)req * a.hq + head) * DH;
      // ALiBi: the key at local position j sits at Delta + j, so the query's
      // distance is measured from q_pos - Delta
      qp[b] = a.q_pos[req] - delta[b];
      orow[b] = req * a.hq + head;
      pslot[b] = d.slot_base + slot + chunk;
      slope2[b] = (KIND == kAlibi) ? a.slopes[head] * kLog2e : 0.f;
      if (KIND == kAlibi) delta[b] = 0;
    }
    // a Delta the table cannot serve is never looked up: its rows turn NaN
    bool bad[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      bad[b] = KIND != kAlibi && a.cos_sin != nullptr && (delta[b] < 0 || delta[b] >= a.max_pos);
      if (bad[b]) delta[b] = 0;
    }
    rotate_query_rows<T, DH, KIND, RB>(qr[0], qptr, a, delta, g, active_blocks);
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if (!bad[b]) continue;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int t = 0; t < 8; ++t) qr[0][b][c][t] = E::from_f(__builtin_nanf(""));
    }
    cur_delta[0] = cur_delta[1] = 0;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      m_run[b] = -INFINITY;
      l_run[b] = 0.f;
#pragma unroll
      for (int n = 0; n < NV; ++n) acc[b][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // Raw words of tiles ia, ia+1 (request-relative; ia+1 may be past the
  // split's end se: it then repeats ia and is dropped by decode_pair).
  __device__ __forceinline__ void fetch_words(int ia, int se, uint64_t& w0, uint64_t& w1) const {
    w0 = a.tiles[t0 + ia];
    w1 = a.tiles[t0 + min(ia + 1, se - 1)];
  }

  __device__ __forceinline__ Pair read_pair(int ia, int se) const {
    uint64_t w0, w1;
    fetch_words(ia, se, w0, w1);
    return decode_pair(ia, se, w0, w1);
  }

  // Split the words by shifts, with device-side guards.
  __device__ __forceinline__ Pair decode_pair(int ia, int se, uint64_t w0, uint64_t w1) const {
    Pair pr;
    pr.mt[0] = unpack_word(w0);
    pr.mt[1] = unpack_word(w1);
    if (ia + 1 >= se) pr.mt[1].mask = 0u;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      pr.priv[x] = ia + x >= nctx;
      if (pr.mt[x].block >= a.num_blocks || pr.mt[x].block < 0) {  // never dereference outside the pool
        pr.mt[x].block = 0;
        pr.mt[x].mask = 0u;
      }
      pr.delta[x] = (kRot && !pr.priv[x]) ? pr.mt[x].offset : 0;
      if (kRot && a.cos_sin != nullptr && pr.delta[x] >= a.max_pos) {  // outside the table: drop the tile
        pr.mt[x].mask = 0u;
        pr.delta[x] = -1;  // "keep the current rotation"
      }
    }
    return pr;
  }

  // Issue every K and V fragment load of a pair.
  __device__ __forceinline__ void load(const Pair& pr, Frags& f) const {
    const T* kc = reinterpret_cast<const T*>(a.k_cache);
    const T* vc = reinterpret_cast<const T*>(a.v_cache);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int64_t base = ((int64_t)pr.mt[x].block * a.hkv + kvh) * (int64_t)(kBlock * DH);
      const T* kp = kc + base + r * DH + 8 * g;
      const T* vp = vc + base + r * kBlock + 4 * g;
#pragma unroll
      for (int c = 0; c < NC; ++c) f.k[x][c] = load8<T>(kp + 32 * c);
#pragma unroll
      for (int n = 0; n < NV; ++n) f.v[x][n] = load4_stream<T>(vp + n * 16 * kBlock);
    }
  }

  // Single relative rotation of the query when a tile's document changes.
  __device__ __forceinline__ void rotate_for(const Pair& pr) {
    if (!kRot) return;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      if (pr.delta[x] >= 0 && pr.delta[x] != cur_delta[x]) {
        rotate_query<T, DH, KIND, RB>(qr[x * (NQ - 1)], qptr, a, pr.delta[x], g, active_blocks);
        cur_delta[x] = pr.delta[x];
      }
    }
  }

  // Scores S^T[key 4g+j][row r] of tile x of a pair.
  __device__ __forceinline__ void scores(const F8 (&k)[NC], int qset, f32x4 (&s)[RB]) const {
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      // unconditional: a predicated product lets the compiler sink (and
      // serialise) the K loads feeding it
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) z = E::mma(k[c], qr[qset][b][c], z);
      s[b] = z;
    }
  }

  // Scores, mask, online softmax and P V of one pair.
  __device__ __forceinline__ void consume(const Pair& pr, Frags& f) {
    f32x4 s[2][RB];
#pragma unroll
    for (int x = 0; x < 2; ++x) scores(f.k[x], x * (NQ - 1), s[x]);
    softmax_pv(pr, f.v, s);
  }

  // Mask, online softmax and P V of one pair whose scores are computed.
  __device__ __forceinline__ void softmax_pv(const Pair& pr, F4 (&fv)[2][NV], const f32x4 (&s)[2][RB]) {
    // zero V of empty slots (partial blocks, dropped tiles): never multiply garbage
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      if (pr.mt[x].mask != 0xFFFFu) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool ok = (pr.mt[x].mask >> (4 * g + j)) & 1u;
#pragma unroll
          for (int n = 0; n < NV; ++n) fv[x][n][j] = ok ? fv[x][n][j] : E::from_f(0.f);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if (b >= active_blocks) continue;
      float sv[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int slot = 4 * g + j;
          bool ok = (pr.mt[x].mask >> slot) & 1u;
          const int kpos = pr.mt[x].offset + slot;
          if (PREFILL && pr.priv[x]) ok = ok && (kpos <= qp[b]);
          float v = s[x][b][j] * a.scale_log2;
          if (KIND == kAlibi) v += slope2[b] * (float)(kpos - qp[b]);
          v = ok ? v : -INFINITY;
          sv[x][j] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = xor_max16_32(mx);
      // Lazy rescale: the reference max m_run only moves (and acc, l are
      // rescaled) when some row's max exceeds it by more than 2^SLACK, so
      // every probability stays <= 2^SLACK; exact in real arithmetic, and the
      // combine uses the same reference.
      if (__any(mx > m_run[b] + (float)LAZY_RESCALE_SLACK)) {
        const float m_new = fmaxf(m_run[b], mx);
        const float alpha = (m_run[b] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[b] - m_new);
        l_run[b] *= alpha;
#pragma unroll
        for (int n = 0; n < NV; ++n) acc[b][n] *= alpha;
        m_run[b] = m_new;
      }
      const float m_use = (m_run[b] == -INFINITY) ? 0.f : m_run[b];
      F8 pf;
      float psum = 0.f;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pj = __builtin_amdgcn_exp2f(sv[x][j] - m_use);
          psum += pj;
          pf[4 * x + j] = E::from_f(pj);
        }
      }
      l_run[b] += psum;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        F8 v8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v8[j] = fv[0][n][j];
          v8[4 + j] = fv[1][n][j];
        }
        acc[b][n] = E::mma(v8, pf, acc[b][n]);
      }
    }
  }

  // O[row r][16n + 4g + j] = acc[b][n][j]: normalised output (one split) or an
  // unnormalised (m, l, acc) partial.
  __device__ __forceinline__ void finalize(int split) {
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if (b >= active_blocks) continue;
      const float l_tot = xor_sum16_32(l_run[b]);
      if (!rvalid[b]) continue;
      if (a.num_splits == 1 && !a.force_partials && pslot[b] < 0) {
        const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
        T* o = reinterpret_cast<T*>(a.out) + (int64_t)orow[b] * DH + 4 * g;
#pragma unroll
        for (int n = 0; n < NV; ++n) {
          F4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = E::from_f(acc[b][n][j] * inv);
          *reinterpret_cast<F4*>(o + 16 * n) = w;
        }
      } else {
        const int64_t prow = (int64_t)(pslot[b] >= 0 ? pslot[b] : split) * a.rows_bound + orow[b];
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
};

// Splits used by a request of nt tiles: one per `chunk` tiles (at least one,
// at most the grid's extent; the last split takes any remainder).
__device__ __forceinline__ int request_splits(int nt, int chunk, int max_splits) {
  return max(1, min(max_splits, (nt + chunk - 1) / chunk));
}

// This split's share of a request's tiles: [sb, se).  Returns false for a
// split the request does not use.
__device__ __forceinline__ bool split_range(int nt, int chunk, int max_splits, int split, int& sb, int& se) {
  const int ns = request_splits(nt, chunk, max_splits);
  if (split >= ns) return false;
  sb = min(nt, split * chunk);
  se = (split == ns - 1) ? nt : min(nt, sb + chunk);
  return true;
}

// Launches the LDS-staged bf16 prefill kernel (prefill_lds.hip); returns
// hipErrorNotSupported for shapes it does not cover.
hipError_t launch_prefill_lds(const AttnArgs& a, int kind, bool defer, int head_dim, int rb, int row_tiles,
                              int splits, int num_reqs, int hkv, hipStream_t st);

// Launches the LDS-staged document pass (bf16; prefill_lds.hip): grid (KV
// head, work item), each item docpass_row_blocks x 16 rows.
hipError_t launch_docpass_lds(const AttnArgs& a, const DocPassArgs& d, int kind, int head_dim, int num_work, int hkv,
                              hipStream_t st);

}  // namespace lazy
