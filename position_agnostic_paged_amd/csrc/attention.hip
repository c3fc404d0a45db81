// Fused paged attention over a position-agnostic KV cache with the document
// offset applied inside the kernel (prefill and decode), plus the split-K
// log-sum-exp combine.
//
// What is computed (LazyAttention notes, papernotes.org, "Method: overall
// framework" and "Key designs"; gist.science summary, "Implementazione
// Tecnica"): for every query row, softmax(scale * q . k' + bias) V over the
// request's tiles, where k' is the key at its global position.  Cached
// document keys are stored rotated at document-local positions, so
// k' = R_Delta k_cached; the kernel applies the equivalent single relative
// rotation to the query, q' = R_{-Delta} q, because (R_{-D} q) . k =
// q . (R_D k) exactly (RoPE relativity, notes "Background and motivation").
//
// MI355X design (differs from the pages' Triton kernels, see the design doc):
//   * One kernel for prefill and decode.  Query rows are GQA-packed: the G
//     query heads of a KV head (x the query tokens in prefill) form the
//     16-wide column blocks of the MFMA products, so a K/V tile is read once
//     for all G heads (notes, "Generality": GQA/MQA need no change).
//   * S^T = K Q'^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16: the K
//     cache is token-major and the V cache channel-major inside a block, so
//     both operands load straight from HBM with 16-byte (K) / 8-byte (V)
//     coalesced loads, no LDS staging, and the score layout out of the first
//     product is exactly the B operand of the second.
//   * The query is re-rotated only when the tile's Delta changes, i.e. once
//     per document, in prefill and decode alike (the notes' decode rule;
//     in prefill it replaces the per-tile K rotation of the pages' kernel:
//     on gfx950 a VALU rotation of every K tile costs more issue slots than
//     the tile's MFMA work, while one query rotation per document is ~1/L of
//     that).  Each lane owns whole rotation pairs, so rotation is lane-local.
//   * The tile word (block, offset, mask) is one wave-uniform 8-byte load,
//     split with shifts; no block-table, offset or mask arrays are read.
//   * Split-K over tiles: every (request, KV head, row tile, split) wave
//     writes (m, l, acc) partials when more than one split is used.
//   * Masked slots are selected to -inf (never multiplied) and their V
//     values to 0, so garbage in unused slots of partial blocks cannot leak.
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
// Uneven lengths: four rounds, so the dispatcher can balance waves that
// progress at different speeds (measured on MI355X: 64 x 32K uniform batch
// best at 2048, 48 x 8K-66K batch best at 8192).
#ifndef LAZY_DECODE_WAVE_TARGET
#define LAZY_DECODE_WAVE_TARGET 2048
#endif
#ifndef LAZY_DECODE_WAVE_TARGET_UNEVEN
#define LAZY_DECODE_WAVE_TARGET_UNEVEN 8192
#endif
// Prefill split heuristic: about this many workgroups per launch.
#ifndef LAZY_PREFILL_WG_TARGET
#define LAZY_PREFILL_WG_TARGET 512
#endif
// 1: wave index through readfirstlane (tile words via the scalar cache);
// 0: plain thread index (tile words via vector loads), measured faster.
#ifndef LAZY_UNIFORM_WAVE
#define LAZY_UNIFORM_WAVE 0
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
};

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

// Per-wave attention state: RB blocks of 16 query rows of one (request, KV
// head) against a stream of tile pairs.  Shared by the prefill and decode
// kernels.  Query row rho of a request is (token rho / G, head kvh*G + rho % G).
template <typename T, int DH, int KIND, bool DEFER, bool PREFILL, int RB>
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
  static constexpr int NQ = kRot ? 2 : 1;

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
      for (int n = 0; n < NV; ++n) f.v[x][n] = load4<T>(vp + n * 16 * kBlock);
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

  // Scores, mask, online softmax and P V of one pair.
  __device__ __forceinline__ void consume(const Pair& pr, Frags& f) {
    f32x4 s[2][RB];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        // unconditional: a predicated product lets the compiler sink (and
        // serialise) the K loads feeding it
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) z = E::mma(f.k[x][c], qr[x * (NQ - 1)][b][c], z);
        s[x][b] = z;
      }
    }
    // zero V of empty slots (partial blocks, dropped tiles): never multiply garbage
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      if (pr.mt[x].mask != 0xFFFFu) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool ok = (pr.mt[x].mask >> (4 * g + j)) & 1u;
#pragma unroll
          for (int n = 0; n < NV; ++n) f.v[x][n][j] = ok ? f.v[x][n][j] : E::from_f(0.f);
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
          v8[j] = f.v[0][n][j];
          v8[4 + j] = f.v[1][n][j];
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
      if (a.num_splits == 1) {
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
        const int64_t prow = (int64_t)split * a.rows_bound + orow[b];
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

// Prefill: one wave = RB blocks of 16 query rows x one split of the request's
// tiles; a workgroup = WR waves over consecutive row blocks (same split).
template <typename T, int DH, int KIND, bool DEFER, int RB, int WR>
__global__ __launch_bounds__(64 * WR) void prefill_kernel(AttnArgs a) {
  using W = WaveAttn<T, DH, KIND, DEFER, true, RB>;
  const int lane = threadIdx.x & 63;
#if LAZY_UNIFORM_WAVE
  const int wr = uniform(threadIdx.x >> 6);  // wave-uniform: keeps tile metadata in scalar registers
#else
  const int wr = threadIdx.x >> 6;
#endif
  const int req = blockIdx.z;
  const int kvh = blockIdx.y;
  const int row_tile = blockIdx.x / a.num_splits;
  const int split = blockIdx.x % a.num_splits;

  const int q0 = a.q_start[req];
  int nq = a.q_start[req + 1] - q0;
  // never address query rows beyond what the grid and workspace were sized for
  nq = min(nq, a.max_q_len);
  nq = max(0, min(nq, a.rows_bound / a.hq - q0));
  const int nrows = nq * a.group;
  const int rb0 = (row_tile * WR + wr) * RB;
  if (rb0 * 16 >= nrows) return;  // no rows for this wave (no barriers follow)

  const int nt = a.tile_start[req + 1] - a.tile_start[req];
  int sb, se;
  if (!split_range(nt, a.chunk, a.num_splits, split, sb, se)) return;  // unused split (no barriers follow)
  W w(a, lane, kvh, req, q0, nrows, rb0, a.q_pos[req]);
  const int npairs = (se - sb + 1) >> 1;
  for (int p = 0; p < npairs; ++p) {
    const typename W::Pair pr = w.read_pair(sb + 2 * p, se);
    typename W::Frags f;
    w.load(pr, f);
    w.rotate_for(pr);
    w.consume(pr, f);
  }
  w.finalize(split);
}

// Decode: one wave = the G query heads of one (request, KV head) x one split;
// a workgroup = WT waves on WT consecutive splits.  Software-pipelined: the
// next pair's K/V loads are in flight while the current pair is consumed.
template <typename T, int DH, int KIND, bool DEFER, int RB, int WT>
__global__ __launch_bounds__(64 * WT) void decode_kernel(AttnArgs a) {
  using W = WaveAttn<T, DH, KIND, DEFER, false, RB>;
  const int lane = threadIdx.x & 63;
#if LAZY_UNIFORM_WAVE
  const int wt = uniform(threadIdx.x >> 6);  // wave-uniform: keeps tile metadata in scalar registers
#else
  const int wt = threadIdx.x >> 6;
#endif
  const int req = blockIdx.z;
  const int kvh = blockIdx.y;
  const int split = blockIdx.x * WT + wt;
  const int nt = a.tile_start[req + 1] - a.tile_start[req];
  int sb, se;
  if (!split_range(nt, a.chunk, a.num_splits, split, sb, se)) return;  // unused split (no barriers follow)

  W w(a, lane, kvh, req, req, a.group, 0, a.q_pos[req]);
  const int npairs = (se - sb + 1) >> 1;
#if LAZY_DECODE_PIPELINE
  if (npairs > 0) {
    typename W::Pair pa = w.read_pair(sb, se), pb;
    typename W::Frags fa, fb;
    w.load(pa, fa);
    for (int p = 0;; p += 2) {
      const bool more = p + 1 < npairs;
      if (more) {
        pb = w.read_pair(sb + 2 * (p + 1), se);
        w.load(pb, fb);
      }
      w.rotate_for(pa);
      w.consume(pa, fa);
      if (!more) break;
      const bool more2 = p + 2 < npairs;
      if (more2) {
        pa = w.read_pair(sb + 2 * (p + 2), se);
        w.load(pa, fa);
      }
      w.rotate_for(pb);
      w.consume(pb, fb);
      if (!more2) break;
    }
  }
#else
  // the next pair's tile words are fetched one iteration ahead
  uint64_t w0 = 0, w1 = 0;
  if (npairs > 0) w.fetch_words(sb, se, w0, w1);
  for (int p = 0; p < npairs; ++p) {
    const typename W::Pair pr = w.decode_pair(sb + 2 * p, se, w0, w1);
    if (p + 1 < npairs) w.fetch_words(sb + 2 * (p + 1), se, w0, w1);
    w.rotate_for(pr);
    typename W::Frags f;
    w.load(pr, f);
    w.consume(pr, f);
  }
#endif
  w.finalize(split);
}

// Split-K combine (flash-decoding): for every output row,
//   M = max_s m_s,  out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,
// over the splits its request used.  Splits that saw no visible key carry
// m = -inf and contribute nothing.
template <typename T, int DH>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, T* __restrict__ out,
                                                      const int32_t* __restrict__ q_start,
                                                      const int32_t* __restrict__ tile_start, int32_t num_reqs,
                                                      int32_t hq, int32_t rows_bound, int32_t max_splits,
                                                      int32_t chunk) {
  constexpr int TPR = DH / 4;  // threads per row, 4 channels each
  const int row = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c4 = (threadIdx.x % TPR) * 4;
  const int rows = min(rows_bound, (q_start != nullptr) ? q_start[num_reqs] * hq : num_reqs * hq);
  if (row >= rows) return;
  int req;
  const int qrow = row / hq;
  if (q_start == nullptr) {
    req = qrow;  // decode: one query row per request
  } else {       // prefill: the request whose row range holds qrow
    int lo = 0, hi = num_reqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (q_start[mid] <= qrow) lo = mid; else hi = mid - 1;
    }
    req = lo;
  }
  const int ns = request_splits(tile_start[req + 1] - tile_start[req], chunk, max_splits);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part_ml[((int64_t)s * rows_bound + row) * 2]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ns; ++s) {
    const int64_t pr = (int64_t)s * rows_bound + row;
    const float w = __builtin_amdgcn_exp2f(part_ml[pr * 2] - Mu);
    L += w * part_ml[pr * 2 + 1];
    const f32x4 v = *reinterpret_cast<const f32x4*>(part_o + pr * DH + c4);
    o += w * v;
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  using F4 = typename Elem<T>::Frag4;
  F4 w4;
#pragma unroll
  for (int j = 0; j < 4; ++j) w4[j] = Elem<T>::from_f(o[j] * inv);
  *reinterpret_cast<F4*>(out + (int64_t)row * DH + c4) = w4;
}

__global__ void debug_unpack_kernel(const uint64_t* w, int64_t n, int32_t* blk, int32_t* off, int32_t* msk) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const TileMeta t = unpack_word(w[i]);
  blk[i] = t.block;
  off[i] = t.offset;
  msk[i] = (int32_t)t.mask;
}

// ------------------------------------------------------------------ host side

namespace {

constexpr int kPrefillRB = 2, kPrefillWR = 4;  // 128 query rows per workgroup
constexpr int kDecodeWT = 4;                   // 4 waves = 4 splits per workgroup

int decode_rb(int group) { return group <= 16 ? 1 : group <= 32 ? 2 : group <= 64 ? 4 : 8; }

struct Plan {
  int rb, wr, wt;
  int row_tiles;
  int splits;  // grid extent along splits
  int chunk;   // tiles per split
  int rows_bound;
};

// Tiles per split so that about `target` work items (waves for decode,
// workgroups for prefill) cover total_tiles x (KV heads x row tiles); each
// request then uses ceil(its tiles / chunk) splits, which balances requests of
// very different lengths.  total_tiles <= 0 means "unknown" (num_reqs x max_tiles).
void size_splits(Plan& p, long per_tile_units, int num_reqs, int max_tiles, int64_t total_tiles, long target,
                 int min_chunk) {
  const long T = total_tiles > 0 ? (long)total_tiles : (long)num_reqs * max_tiles;
  long chunk = (T * per_tile_units + target - 1) / std::max(1L, target);
  chunk = std::max<long>(chunk, min_chunk);
  const int max_splits = 256;
  if ((max_tiles + chunk - 1) / chunk > max_splits) chunk = (max_tiles + max_splits - 1) / max_splits;
  chunk = (chunk + 1) & ~1L;  // whole tile pairs
  p.chunk = (int)std::min<long>(chunk, 1 << 30);
  p.splits = std::max(1, (int)((max_tiles + p.chunk - 1) / p.chunk));
}

Plan make_plan(const lazy_geom* g, int num_reqs, int max_q_len, int max_tiles, int64_t total_tiles, bool prefill) {
  Plan p;
  const int group = g->num_q_heads / g->num_kv_heads;
  if (prefill) {
    p.rb = kPrefillRB;
    p.wr = kPrefillWR;
    p.wt = 1;
    const int rows = max_q_len * group;
    p.row_tiles = (rows + 16 * p.rb * p.wr - 1) / (16 * p.rb * p.wr);
    size_splits(p, (long)g->num_kv_heads * p.row_tiles, num_reqs, max_tiles, total_tiles, LAZY_PREFILL_WG_TARGET, 16);
    p.rows_bound = max_q_len * num_reqs * g->num_q_heads;
  } else {
    p.rb = decode_rb(group);
    p.wr = 1;
    p.wt = kDecodeWT;
    p.row_tiles = 1;
    const bool uneven = total_tiles > 0 && (double)max_tiles * num_reqs > 1.25 * (double)total_tiles;
    size_splits(p, g->num_kv_heads, num_reqs, max_tiles, total_tiles,
                uneven ? LAZY_DECODE_WAVE_TARGET_UNEVEN : LAZY_DECODE_WAVE_TARGET, 32);
    p.rows_bound = num_reqs * g->num_q_heads;
  }
  return p;
}

size_t ws_bytes_for(const lazy_geom* g, const Plan& p) {
  if (p.splits == 1) return 0;
  const size_t per = (size_t)g->head_dim + 2;
  return (size_t)p.splits * (size_t)p.rows_bound * per * sizeof(float) + 256;
}

template <typename T, int DH, int KIND, bool DEFER, int RB>
hipError_t launch_decode(const AttnArgs& a, const Plan& p, int num_reqs, int hkv, hipStream_t st) {
  dim3 grid((unsigned)((p.splits + kDecodeWT - 1) / kDecodeWT), (unsigned)hkv, (unsigned)num_reqs);
  hipLaunchKernelGGL((decode_kernel<T, DH, KIND, DEFER, RB, kDecodeWT>), grid, dim3(64 * kDecodeWT), 0, st, a);
  return hipGetLastError();
}

template <typename T, int DH, int KIND, bool DEFER, bool PREFILL>
hipError_t dispatch_rb(const AttnArgs& a, const Plan& p, int num_reqs, int hkv, hipStream_t st) {
  if (PREFILL) {
    dim3 grid((unsigned)(p.row_tiles * p.splits), (unsigned)hkv, (unsigned)num_reqs);
    hipLaunchKernelGGL((prefill_kernel<T, DH, KIND, DEFER, kPrefillRB, kPrefillWR>), grid, dim3(64 * kPrefillWR), 0,
                       st, a);
    return hipGetLastError();
  }
  switch (p.rb) {
    case 1:
      return launch_decode<T, DH, KIND, DEFER, 1>(a, p, num_reqs, hkv, st);
    case 2:
      return launch_decode<T, DH, KIND, DEFER, 2>(a, p, num_reqs, hkv, st);
    case 4:
      return launch_decode<T, DH, KIND, DEFER, 4>(a, p, num_reqs, hkv, st);
    default:
      return launch_decode<T, DH, KIND, DEFER, 8>(a, p, num_reqs, hkv, st);
  }
}

template <typename T, int DH, bool PREFILL>
hipError_t dispatch_kind(int kind, bool defer, const AttnArgs& a, const Plan& p, int num_reqs, int hkv,
                         hipStream_t st) {
  switch (kind) {
    case kHalf:
      return defer ? dispatch_rb<T, DH, kHalf, true, PREFILL>(a, p, num_reqs, hkv, st)
                   : dispatch_rb<T, DH, kHalf, false, PREFILL>(a, p, num_reqs, hkv, st);
    case kInter:
      return defer ? dispatch_rb<T, DH, kInter, true, PREFILL>(a, p, num_reqs, hkv, st)
                   : dispatch_rb<T, DH, kInter, false, PREFILL>(a, p, num_reqs, hkv, st);
    default:
      return dispatch_rb<T, DH, kAlibi, false, PREFILL>(a, p, num_reqs, hkv, st);
  }
}

template <typename T, int DH>
hipError_t launch_combine(const AttnArgs& a, const Plan& p, const int32_t* q_start, int num_reqs, hipStream_t st) {
  constexpr int rows_per_block = 256 / (DH / 4);
  const int rows = p.rows_bound;
  dim3 grid((unsigned)((rows + rows_per_block - 1) / rows_per_block));
  hipLaunchKernelGGL((combine_kernel<T, DH>), grid, dim3(256), 0, st, a.part_o, a.part_ml,
                     reinterpret_cast<T*>(a.out), q_start, a.tile_start, num_reqs, a.hq, p.rows_bound, p.splits,
                     p.chunk);
  return hipGetLastError();
}

template <bool PREFILL>
hipError_t run(const lazy_geom* g, const lazy_pos_desc* pd, AttnArgs& a, const Plan& p, int num_reqs,
               const int32_t* q_start, hipStream_t st) {
  const bool defer = !(pd->flags & LAZY_FLAG_PREROTATED);
  const int hkv = g->num_kv_heads;
  hipError_t e;
  if (g->dtype == LAZY_BF16) {
    e = (g->head_dim == 128) ? dispatch_kind<bf16, 128, PREFILL>(pd->kind, defer, a, p, num_reqs, hkv, st)
                             : dispatch_kind<bf16, 64, PREFILL>(pd->kind, defer, a, p, num_reqs, hkv, st);
  } else {
    e = (g->head_dim == 128) ? dispatch_kind<float, 128, PREFILL>(pd->kind, defer, a, p, num_reqs, hkv, st)
                             : dispatch_kind<float, 64, PREFILL>(pd->kind, defer, a, p, num_reqs, hkv, st);
  }
  if (e != hipSuccess || p.splits == 1) return e;
  const int32_t* qs = PREFILL ? q_start : nullptr;
  if (g->dtype == LAZY_BF16)
    return (g->head_dim == 128) ? launch_combine<bf16, 128>(a, p, qs, num_reqs, st)
                                : launch_combine<bf16, 64>(a, p, qs, num_reqs, st);
  return (g->head_dim == 128) ? launch_combine<float, 128>(a, p, qs, num_reqs, st)
                              : launch_combine<float, 64>(a, p, qs, num_reqs, st);
}

lazy_status common_checks(const lazy_geom* g, const lazy_pos_desc* pd, const void* kc, const void* vc,
                          int64_t num_blocks, const uint64_t* tiles, const int32_t* tile_start,
                          const int32_t* ctx_tiles, const void* q, const int32_t* qpos, int32_t num_reqs,
                          int32_t max_tiles, void* out) {
  lazy_status st = check_geom(g);
  if (st != LAZY_OK) return st;
  st = check_pos(g, pd);
  if (st != LAZY_OK) return st;
  if (num_reqs < 0) return fail(LAZY_ERR_ARG, "num_reqs must be >= 0 (got %d)", num_reqs);
  if (max_tiles < 0) return fail(LAZY_ERR_ARG, "max_tiles must be >= 0 (got %d)", max_tiles);
  if (num_blocks < 1 || num_blocks > (int64_t)LAZY_MAX_BLOCK_ID + 1)
    return fail(LAZY_ERR_ARG, "num_blocks must be in [1, 2^24] (got %lld)", (long long)num_blocks);
  if (num_reqs > 0 && (!kc || !vc || !tiles || !tile_start || !ctx_tiles || !q || !qpos || !out))
    return fail(LAZY_ERR_ARG, "a required device pointer is NULL");
  if (num_reqs > 65535) return fail(LAZY_ERR_UNSUPPORTED, "num_reqs > 65535 is not supported");
  return LAZY_OK;
}

}  // namespace
}  // namespace lazy

using namespace lazy;

extern "C" size_t lazy_attn_workspace_size(const lazy_geom* geom, int32_t num_reqs, int32_t max_q_len,
                                           int32_t max_tiles, int64_t total_tiles, int32_t is_prefill) {
  if (check_geom(geom) != LAZY_OK || num_reqs <= 0 || max_tiles < 0) return 0;
  if (is_prefill && max_q_len <= 0) return 0;
  const Plan p = make_plan(geom, num_reqs, is_prefill ? max_q_len : 1, max_tiles, total_tiles, is_prefill != 0);
  return ws_bytes_for(geom, p);
}

extern "C" lazy_status lazy_attn_prefill(const lazy_geom* geom, const lazy_pos_desc* pos, const void* k_cache,
                                         const void* v_cache, int64_t num_blocks, const uint64_t* tiles,
                                         const int32_t* tile_start, const int32_t* ctx_tiles, const void* q,
                                         const int32_t* q_start, const int32_t* q_pos0, int32_t num_reqs,
                                         int32_t max_q_len, int32_t max_tiles, int64_t total_tiles, void* out,
                                         void* workspace,
                                         size_t ws_bytes, void* stream) {
  clear_error();
  lazy_status st = common_checks(geom, pos, k_cache, v_cache, num_blocks, tiles, tile_start, ctx_tiles, q, q_pos0,
                                 num_reqs, max_tiles, out);
  if (st != LAZY_OK) return st;
  if (num_reqs > 0 && !q_start) return fail(LAZY_ERR_ARG, "q_start is NULL");
  if (max_q_len < 0) return fail(LAZY_ERR_ARG, "max_q_len must be >= 0 (got %d)", max_q_len);
  if (num_reqs == 0 || max_q_len == 0) return LAZY_OK;
  const int group = geom->num_q_heads / geom->num_kv_heads;
  if ((int64_t)max_q_len * num_reqs * geom->num_q_heads > (int64_t)INT32_MAX / 2 ||
      (int64_t)max_q_len * group > (int64_t)INT32_MAX / 2)
    return fail(LAZY_ERR_UNSUPPORTED, "too many query rows");
  const Plan p = make_plan(geom, num_reqs, max_q_len, max_tiles, total_tiles, true);
  const size_t need = ws_bytes_for(geom, p);
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(LAZY_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  AttnArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.tiles = tiles;
  a.tile_start = tile_start;
  a.ctx_tiles = ctx_tiles;
  a.q = q;
  a.q_start = q_start;
  a.q_pos = q_pos0;
  a.cos_sin = pos->cos_sin;
  a.inv_freq = pos->inv_freq;
  a.max_pos = pos->max_pos;
  a.slopes = pos->alibi_slopes;
  a.scale_log2 = pos->softmax_scale * kLog2e;
  a.out = out;
  a.num_splits = p.splits;
  a.chunk = p.chunk;
  a.hq = geom->num_q_heads;
  a.hkv = geom->num_kv_heads;
  a.group = group;
  a.rows_bound = p.rows_bound;
  a.max_q_len = max_q_len;
  if (need > 0) {
    a.part_o = reinterpret_cast<float*>(workspace);
    a.part_ml = a.part_o + (size_t)p.splits * p.rows_bound * geom->head_dim;
  }
  const hipError_t e = run<true>(geom, pos, a, p, num_reqs, q_start, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LAZY_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return LAZY_OK;
}

extern "C" lazy_status lazy_attn_decode(const lazy_geom* geom, const lazy_pos_desc* pos, const void* k_cache,
                                        const void* v_cache, int64_t num_blocks, const uint64_t* tiles,
                                        const int32_t* tile_start, const int32_t* ctx_tiles, const void* q,
                                        const int32_t* q_pos, int32_t num_reqs, int32_t max_tiles,
                                        int64_t total_tiles, void* out,
                                        void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  lazy_status st = common_checks(geom, pos, k_cache, v_cache, num_blocks, tiles, tile_start, ctx_tiles, q, q_pos,
                                 num_reqs, max_tiles, out);
  if (st != LAZY_OK) return st;
  if (num_reqs == 0) return LAZY_OK;
  const Plan p = make_plan(geom, num_reqs, 1, max_tiles, total_tiles, false);
  const size_t need = ws_bytes_for(geom, p);
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(LAZY_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  AttnArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.tiles = tiles;
  a.tile_start = tile_start;
  a.ctx_tiles = ctx_tiles;
  a.q = q;
  a.q_start = nullptr;
  a.q_pos = q_pos;
  a.cos_sin = pos->cos_sin;
  a.inv_freq = pos->inv_freq;
  a.max_pos = pos->max_pos;
  a.slopes = pos->alibi_slopes;
  a.scale_log2 = pos->softmax_scale * kLog2e;
  a.out = out;
  a.num_splits = p.splits;
  a.chunk = p.chunk;
  a.hq = geom->num_q_heads;
  a.hkv = geom->num_kv_heads;
  a.group = geom->num_q_heads / geom->num_kv_heads;
  a.rows_bound = p.rows_bound;
  a.max_q_len = 1;
  if (need > 0) {
    a.part_o = reinterpret_cast<float*>(workspace);
    a.part_ml = a.part_o + (size_t)p.splits * p.rows_bound * geom->head_dim;
  }
  const hipError_t e = run<false>(geom, pos, a, p, num_reqs, nullptr, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LAZY_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return LAZY_OK;
}

extern "C" lazy_status lazy_debug_unpack(const uint64_t* words, int64_t n, int32_t* block, int32_t* offset,
                                         int32_t* mask, void* stream) {
  clear_error();
  if (n < 0) return fail(LAZY_ERR_ARG, "n must be >= 0");
  if (n == 0) return LAZY_OK;
  if (!words || !block || !offset || !mask) return fail(LAZY_ERR_ARG, "a device pointer is NULL");
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(debug_unpack_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), words,
                     n, block, offset, mask);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(LAZY_ERR_HIP, "unpack launch failed: %s", hipGetErrorString(e));
  return LAZY_OK;
}
